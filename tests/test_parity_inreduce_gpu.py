"""The in-kernel reduction of two K splits (the second split to finish adds the
first's partial and stores the tile), on the GPU, through the C ABI.

"A Blackwell GEMM by Hand in CuTe DSL", section 9: split-K for decode shapes.
With two splits IEEE addition is commutative, so the result must be bitwise
the one of the second-pass reduction (GEMM_INREDUCE=0), whichever split
finishes second; on small integers bitwise the oracle's; and the per-tile
counters must be back at zero after every call, so repeated calls (and calls
of other shapes in between) give the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_inputs import make_operands
from tests.gpu_util import compare_full, new_handle, run_gpu, say, TORCH_DT

pytestmark = pytest.mark.gpu

CONFIGS = ["256x256x64_w8_pp2", "256x128x64_w4_u8"]


@pytest.mark.parametrize("config", CONFIGS)
@pytest.mark.parametrize("M,N,K", [(256, 1024, 2048), (300, 700, 1000), (513, 260, 136)])
def test_two_splits_small_integers_bitwise(config, M, N, K):
    say("case in-kernel 2-split int3 %s M=%d N=%d K=%d" % (config, M, N, K))
    h = new_handle(config, 2)
    A, B = make_operands(M, N, K, "bf16", "int3", seed=M + N, lda=K + 8, ldb=K + 16)
    Cr, _ = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    for _ in range(2):                                    # counters reset between calls
        C = run_gpu(h, A, B, K, "bf16", "fp32")
        assert np.array_equal(C, Cr)
    h.close()


@pytest.mark.parametrize("config", CONFIGS)
@pytest.mark.parametrize("M,N,K,outd", [(256, 28672, 8192, "bf16"), (257, 1100, 4096, "fp32"),
                                        (200, 2048, 1024, "fp16")])
def test_two_splits_equal_second_pass_bitwise(config, M, N, K, outd):
    say("case in-kernel vs second pass %s M=%d N=%d K=%d ->%s" % (config, M, N, K, outd))
    A, B = make_operands(M, N, K, "bf16", "llm", seed=K)
    h1 = new_handle(config, 2, inreduce=1)
    h0 = new_handle(config, 2, inreduce=0)
    C1 = run_gpu(h1, A, B, K, "bf16", outd)
    C0 = run_gpu(h0, A, B, K, "bf16", outd)
    assert np.array_equal(C1, C0)
    C1b = run_gpu(h1, A, B, K, "bf16", outd)
    assert np.array_equal(C1b, C1)
    if M * N * K <= 2 ** 31:
        compare_full(C1, A, B, K, "bf16", outd, "in-kernel 2 splits")
    h1.close()
    h0.close()


def test_default_decode_plan_is_reduced_in_kernel_and_matches_oracle():
    import dense_gemm_nt_amd as g
    M, N, K = 256, 28672, 8192
    p = g.gemm_plan(M, N, K, 0, 0)
    assert p["inreduce"] == 1 and p["splits"] == 2
    say("case default decode MLP-up plan %s, in-kernel reduction" % p["name"])
    h = new_handle()
    A, B = make_operands(M, N, K, "bf16", "llm", seed=0)
    C = run_gpu(h, A, B, K, "bf16", "bf16")
    compare_full(C, A, B, K, "bf16", "bf16", "decode MLP-up")
    h.close()


def test_fused_epilogue_after_in_kernel_reduction():
    from dense_gemm_nt_amd import _lib
    from oracle import epilogue as oepi
    from tests.tolerance import check_epilogue
    M, N, K = 256, 1536, 2048
    say("case in-kernel reduction + bias/GELU epilogue M=%d N=%d K=%d" % (M, N, K))
    A, B = make_operands(M, N, K, "bf16", "llm", seed=9)
    dev = torch.device("cuda", 0)
    bias = (torch.rand(N, generator=torch.Generator().manual_seed(1)) - 0.5).float()
    for config in CONFIGS:
        h = new_handle(config, 2)
        Ad, Bd, bd = A.to(dev), B.to(dev), bias.to(dev)
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        epi = _lib.epilogue(1.5, 0.0, bd.data_ptr(), "n", "gelu")
        s = torch.cuda.current_stream(dev)
        h.run_raw_ex(Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), M, N, K, K, K, N, 0, 0, epi,
                     s.cuda_stream)
        s.synchronize()
        Cr, S = oracle.gemm_nt(A, B, K=K)
        D = oepi.apply(Cr, alpha=1.5, bias=bias.numpy().astype(np.float64), bias_along="n",
                       act="gelu")
        aS, t = oepi.scale_of(S, alpha=1.5, bias=bias.numpy().astype(np.float64), bias_along="n")
        check_epilogue(C.float().cpu().double().numpy(), D, aS, t, "bf16", config)
        h.close()


# Any number of K splits on the tile kernels (32x128, 128x128 with four
# stages, K-masked): the last split of a tile to finish adds the others'
# partials in split order, so every result must be bitwise the second pass's
# (GEMM_INREDUCE=0), whichever split came last, and stay so over repeated
# calls (the counters go back to zero).
T32, T128, KMASK = "32x128x64_w4_s6", "128x128x64_w8_s4", "128x128x64_w8_s4_kmask"


@pytest.mark.parametrize("config,splits,M,N,K,outd", [
    (T32, 2, 64, 1000, 2048, "bf16"), (T32, 3, 1, 8192, 8192, "bf16"), (T32, 5, 20, 1000, 4104, "fp16"),
    (T32, 6, 16, 4096, 16384, "bf16"), (T32, 12, 1, 2048, 32768, "fp32"), (T32, 7, 33, 300, 1800, "fp32"),
    (T128, 2, 128, 2100, 1024, "bf16"), (T128, 4, 96, 8192, 8192, "bf16"), (T128, 3, 127, 3000, 2056, "fp32"),
    (KMASK, 3, 90, 700, 1001, "bf16")])
def test_tile_kernel_splits_equal_second_pass_bitwise(config, splits, M, N, K, outd):
    say("case tile in-kernel %d splits vs second pass %s M=%d N=%d K=%d ->%s" % (splits, config, M, N, K, outd))
    ld = -(-K // 8) * 8
    A, B = make_operands(M, N, K, "bf16", "llm", seed=K + splits, lda=ld, ldb=ld)
    h1 = new_handle(config, splits, inreduce=1)
    h0 = new_handle(config, splits, inreduce=0)
    C1 = run_gpu(h1, A, B, K, "bf16", outd)
    C0 = run_gpu(h0, A, B, K, "bf16", outd)
    assert np.array_equal(C1, C0)
    for _ in range(2):
        assert np.array_equal(run_gpu(h1, A, B, K, "bf16", outd), C1)
    if M * N * K <= 2 ** 31:
        compare_full(C1, A, B, K, "bf16", outd, "tile in-kernel %d splits" % splits)
    h1.close()
    h0.close()


def test_tile_kernel_splits_small_integers_bitwise():
    M, N, K, splits = 40, 1100, 5000, 9
    say("case tile in-kernel int3 %d splits M=%d N=%d K=%d" % (splits, M, N, K))
    A, B = make_operands(M, N, K, "bf16", "int3", seed=9)
    Cr, _ = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    h = new_handle(T32, splits, inreduce=1)
    for _ in range(2):
        assert np.array_equal(run_gpu(h, A, B, K, "bf16", "fp32"), Cr)
    h.close()


def test_default_small_m_plans_reduce_in_kernel():
    import dense_gemm_nt_amd as g
    for M, N, K in [(1, 8192, 8192), (32, 8192, 8192), (1, 4096, 16384), (96, 8192, 8192)]:
        p = g.gemm_plan(M, N, K, 0, 0)
        assert p["splits"] > 1 and p["inreduce"] == 1, (M, N, K, p)
