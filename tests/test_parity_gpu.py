"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Small and medium shapes compare every output element with the oracle; the
full-size workloads compare whole sampled rows and random points, plus exact
closed forms over the whole output.  Bound: |C - C_ref| <= 1e-3 S + 1e-5
(+ one output ulp for 16-bit outputs), S = sum_k |a b| (tests/tolerance.py).
Small-integer inputs make every partial sum exact, so there the comparison is
bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_inputs import make_operands
from tests.gpu_util import compare_full, compare_sampled, new_handle, run_gpu, say, TORCH_DT

pytestmark = pytest.mark.gpu

CONFIGS = ["128x128x64_w8_s4", "128x128x64_w8_s4_kmask", "256x256x64_w8_pp2",
           "128x128x64_w8_s2", "32x128x64_w4_s6", "256x128x64_w4_u8"]


@pytest.fixture(scope="module")
def h():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return new_handle()


def ld8(x):
    """Smallest leading dimension >= x that keeps rows 16-byte aligned."""
    return (x + 7) // 8 * 8


def _bits(x, dt):
    return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# ------------------------------------------------------------ the small config

def test_small_config_512_bf16_to_fp32(h):
    say("case 512^3 bf16->fp32 uniform seed 0")
    A, B = make_operands(512, 512, 512, "bf16", "uniform", seed=0)
    C = run_gpu(h, A, B, 512, "bf16", "fp32")
    err, worst = compare_full(C, A, B, 512, "bf16", "fp32", "512^3")
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))


# ------------------------------------------------------------ every element

FULL_CASES = [
    # M, N, K, in, out, dist, lda_pad, ldc_pad
    (256, 256, 64, "bf16", "fp32", "uniform", 0, 0),
    (300, 520, 264, "bf16", "bf16", "uniform", 0, 0),
    (257, 129, 72, "fp16", "fp16", "uniform", 8, 3),
    (1000, 4097, 1536, "fp16", "fp32", "uniform", 0, 0),      # ragged config, unaligned ldc
    (1, 8192, 8192, "fp16", "fp32", "uniform", 0, 0),         # ragged config, M = 1
    (64, 64, 16, "bf16", "bf16", "llm", 0, 0),
    (5, 7, 13, "bf16", "fp32", "uniform", 3, 1),              # K % 8 != 0
    (33, 100, 37, "fp16", "bf16", "uniform", 11, 0),          # K % 8 != 0, padded rows
    (130, 70, 1, "bf16", "fp32", "uniform", 7, 0),            # K = 1
    (96, 96, 4104, "bf16", "bf16", "llm", 0, 5),              # long K, split-K plan
]


@pytest.mark.parametrize("M,N,K,ind,outd,dist,pad,cpad", FULL_CASES)
def test_parity_every_element(h, M, N, K, ind, outd, dist, pad, cpad):
    say("case full M=%d N=%d K=%d %s->%s %s lda+%d ldc+%d" % (M, N, K, ind, outd, dist, pad, cpad))
    A, B = make_operands(M, N, K, ind, dist, seed=M + N + K, lda=ld8(K + pad), ldb=ld8(K + 2 * pad))
    C = run_gpu(h, A, B, K, ind, outd, ldc=N + cpad)
    err, worst = compare_full(C, A, B, K, ind, outd, "M=%d N=%d K=%d" % (M, N, K))
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))


# ------------------------------------------------------------ exact integers, every config

@pytest.mark.parametrize("config", CONFIGS)
@pytest.mark.parametrize("splits", [None, 3])
def test_small_integers_bitwise(config, splits):
    # entries in {-3..3}: every partial sum is an integer below 2^24, so any
    # summation order gives the exact result; a lost, repeated or misplaced
    # k-slab or tile changes the bits.
    M, N, K = 300, 280, 1000 if not config.endswith("kmask") else 997
    say("case int3 bitwise config=%s splits=%s M=%d N=%d K=%d" % (config, splits, M, N, K))
    hh = new_handle(config, splits)
    A, B = make_operands(M, N, K, "bf16", "int3", seed=5, lda=ld8(K + 1), ldb=ld8(K + 1))
    C = run_gpu(hh, A, B, K, "bf16", "fp32")
    Cr, _ = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    assert np.array_equal(C, Cr)
    # 16-bit output: the exact sum rounded to nearest even
    Cb = run_gpu(hh, A, B, K, "bf16", "bf16", keep_device=True)
    want = oracle.encode(Cr, "bf16")
    assert np.array_equal(_bits(Cb, torch.bfloat16), want)
    hh.close()


@pytest.mark.parametrize("config", ["256x256x64_w8_pp2", "128x128x64_w8_s4", "256x128x64_w4_u8"])
@pytest.mark.parametrize("K", [8, 64, 128, 192, 200])
def test_short_k_bitwise(config, K):
    # one to four k-slabs: the prologue and drain paths of the multi-slab rings
    M, N = 300, 280
    say("case short-K int3 bitwise config=%s M=%d N=%d K=%d" % (config, M, N, K))
    hh = new_handle(config)
    A, B = make_operands(M, N, K, "bf16", "int3", seed=K, lda=ld8(K + 8), ldb=ld8(K))
    C = run_gpu(hh, A, B, K, "bf16", "fp32")
    Cr, _ = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    assert np.array_equal(C, Cr)
    hh.close()


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("K,outd", [(257, "bf16"), (259, "bf16"), (5000, "bf16"), (5000, "fp16"),
                                    (28672, "bf16"), (1536, "fp32")])
def test_all_ones_gives_rounded_K(h, K, outd):
    say("case all-ones K=%d out=%s" % (K, outd))
    A, B = make_operands(70, 300, K, "bf16", "ones", lda=ld8(K), ldb=ld8(K))
    C = run_gpu(h, A, B, K, "bf16", outd, keep_device=True)
    if outd == "fp32":
        assert bool((C == K).all())
    else:
        want = int(oracle.encode([float(K)], outd)[0])   # 257 -> 256, 259 -> 260, 5000 -> 4992
        got = _bits(C, TORCH_DT[outd])
        assert np.all(got == want), (np.unique(got), want)


@pytest.mark.parametrize("ind", ["bf16", "fp16"])
def test_identity_B_returns_A(h, ind):
    say("case identity %s" % ind)
    K = 384
    A, _ = make_operands(200, K, K, ind, "uniform", seed=9)
    B = torch.eye(K, dtype=TORCH_DT[ind])
    C = run_gpu(h, A, B, K, ind, ind, keep_device=True)
    assert np.array_equal(_bits(C, None), _bits(A, None))


def _rank1(M, N, K, seed):
    # A[i,k] = u_i x_k, B[j,k] = v_j x_k with x_k = +-1 and u, v powers of two:
    # C[i,j] = u_i v_j K exactly (K is a power of two here, exact in bf16 too).
    g = torch.Generator().manual_seed(seed)
    u = torch.exp2(torch.randint(-2, 3, (M,), generator=g).float()) * (torch.randint(0, 2, (M,), generator=g) * 2 - 1)
    v = torch.exp2(torch.randint(-2, 3, (N,), generator=g).float()) * (torch.randint(0, 2, (N,), generator=g) * 2 - 1)
    x = (torch.randint(0, 2, (K,), generator=g) * 2 - 1).float()
    return u, v, x


@pytest.mark.parametrize("M,N,K", [(8192, 28672, 8192), (4096, 4096, 4096), (256, 8192, 28672)])
def test_rank1_whole_output_at_full_size(M, N, K):
    say("case rank-1 full output M=%d N=%d K=%d" % (M, N, K))
    dev = torch.device("cuda", 0)
    u, v, x = _rank1(M, N, K, seed=M + N)
    A = (u[:, None] * x[None, :]).to(torch.bfloat16).to(dev)
    B = (v[:, None] * x[None, :]).to(torch.bfloat16).to(dev)
    hh = new_handle()
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    hh.run_raw(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, K, K, N, 0, 0,
               torch.cuda.current_stream().cuda_stream)
    want = (u[:, None] * v[None, :] * float(K)).to(dev)     # exact: powers of two times 2^13..2^15
    torch.cuda.synchronize()
    assert bool((C.float() == want).all())
    del A, B, C, want
    hh.close()
    torch.cuda.empty_cache()


# ------------------------------------------------------------ the workloads at full size

# Shapes the oracle finishes in a few seconds on the host (60-70 G multiply-adds
# at most): compared with the oracle on every output element.
WORKLOADS_FULL = [
    # M, N, K, in, out, dist
    (4096, 4096, 4096, "bf16", "bf16", "uniform"),
    (4096, 4096, 4096, "fp16", "bf16", "uniform"),
    (4096, 4096, 4096, "fp16", "fp16", "uniform"),
    (256, 28672, 8192, "bf16", "bf16", "llm"),
    (256, 8192, 28672, "bf16", "bf16", "llm"),
    (256, 10240, 8192, "bf16", "bf16", "llm"),
    (256, 8192, 8192, "bf16", "bf16", "llm"),
    (127, 28672, 8192, "fp16", "fp32", "uniform"),
    (3000, 3000, 5000, "fp16", "fp32", "uniform"),
    (1000, 4097, 1536, "fp16", "fp32", "uniform"),
    (1, 8192, 8192, "fp16", "fp32", "uniform"),
]

# The two prefill shapes (550 and 1924 G multiply-adds): whole rows and random
# points against the oracle.
WORKLOADS_SAMPLED = [
    (8192, 8192, 8192, "bf16", "bf16", "llm"),
    (8192, 28672, 8192, "bf16", "bf16", "llm"),
]


@pytest.mark.parametrize("M,N,K,ind,outd,dist", WORKLOADS_FULL)
def test_workloads_every_element(h, M, N, K, ind, outd, dist):
    say("case workload (every element) M=%d N=%d K=%d %s->%s %s" % (M, N, K, ind, outd, dist))
    A, B = make_operands(M, N, K, ind, dist, seed=0)
    C = run_gpu(h, A, B, K, ind, outd)
    err, worst = compare_full(C, A, B, K, ind, outd, "M=%d N=%d K=%d" % (M, N, K))
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))
    del C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,N,K,ind,outd,dist", WORKLOADS_SAMPLED)
def test_workloads_sampled(h, M, N, K, ind, outd, dist):
    say("case workload (sampled) M=%d N=%d K=%d %s->%s %s" % (M, N, K, ind, outd, dist))
    A, B = make_operands(M, N, K, ind, dist, seed=0)
    C = run_gpu(h, A, B, K, ind, outd)
    err, worst = compare_sampled(C, A, B, K, ind, outd, "M=%d N=%d K=%d" % (M, N, K),
                                 n_rows=8, n_points=20000)
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))
    torch.cuda.empty_cache()


# ------------------------------------------------------------ edges, streams, determinism

def test_empty_outputs_do_nothing(h):
    say("case empty M/N")
    dev = torch.device("cuda", 0)
    A = torch.ones((4, 16), dtype=torch.bfloat16, device=dev)
    C = torch.full((4, 8), 7.0, dtype=torch.float32, device=dev)
    h.run_raw(A.data_ptr(), A.data_ptr(), C.data_ptr(), 0, 8, 16, 16, 16, 8, 0, 2, 0)
    h.run_raw(A.data_ptr(), A.data_ptr(), C.data_ptr(), 4, 0, 16, 16, 16, 8, 0, 2, 0)
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())


def test_K_zero_writes_zeros(h):
    say("case K=0")
    dev = torch.device("cuda", 0)
    C = torch.full((70, 90), 7.0, dtype=torch.float32, device=dev)
    h.run_raw(0, 0, C.data_ptr(), 70, 90, 0, 0, 0, 90, 0, 2, 0)
    torch.cuda.synchronize()
    assert bool((C == 0).all())


def test_side_stream_and_repeat_determinism(h):
    say("case side stream + determinism (split-K plan)")
    M, N, K = 256, 8192, 8192
    A, B = make_operands(M, N, K, "bf16", "llm", seed=1)
    s = torch.cuda.Stream()
    C1 = run_gpu(h, A, B, K, "bf16", "fp32", stream=s)
    C2 = run_gpu(h, A, B, K, "bf16", "fp32")
    assert np.array_equal(C1, C2)
    compare_sampled(C1, A, B, K, "bf16", "fp32", "side stream")


def test_large_leading_dimension(h):
    say("case lda near the limit")
    K, lda = 256, (1 << 22) - 8
    A, B = make_operands(16, 200, K, "bf16", "uniform", seed=3, lda=lda, ldb=K + 8)
    C = run_gpu(h, A, B, K, "bf16", "fp32")
    compare_full(C, A, B, K, "bf16", "fp32", "lda=2^22-8")


@pytest.mark.parametrize("config", ["256x256x64_w8_pp2", "256x128x64_w4_u8", "128x128x64_w8_s4"])
@pytest.mark.parametrize("which", ["a", "b"])
def test_largest_leading_dimension_on_the_big_tiles(config, which):
    # lda (or ldb) just below the library's limit on the 256- and 128-row
    # tiles, whose row offsets times the pitch come closest to the 32-bit
    # range of a buffer load's offset and of a tile's buffer size; two tile
    # rows (the second ragged) and a ragged column tile
    M, N, K, ld = 260, 300, 128, (1 << 22) - 8
    say("case ld%s = 2^22-8 on %s M=%d N=%d K=%d" % (which, config, M, N, K))
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=5, lda=ld if which == "a" else K,
                         ldb=ld if which == "b" else K)
    hc = new_handle(config)
    C = run_gpu(hc, A, B, K, "bf16", "fp32")
    hc.close()
    compare_full(C, A, B, K, "bf16", "fp32", "%s ld%s=2^22-8" % (config, which))
    del A, B


def test_output_beyond_two_to_the_31_elements(h):
    # C with more than 2^31 elements (4.3 GB of BF16): the store offsets of its
    # last rows exceed the 32-bit range; rows on both sides of the boundary
    # against the oracle (C stays on the GPU: only those rows come back)
    from tests.tolerance import check
    M, N, K = 65600, 32768, 16
    assert M * N > 2 ** 31
    say("case output past 2^31 elements M=%d N=%d K=%d" % (M, N, K))
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=11)
    dev = torch.device("cuda", 0)
    Ad, Bd = A.to(dev), B.to(dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    h.run_raw(Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), M, N, K, K, K, N, 0, 0, 0)
    torch.cuda.synchronize()
    rows = [0, (2 ** 31) // N - 1, (2 ** 31) // N, M - 1]
    got = C[rows].float().cpu().double().numpy()
    Cr, S = oracle.gemm_nt_rows(A, B, rows, K=K, in_dtype="bf16")
    check(got, Cr, S, "bf16", "rows around 2^31 elements")
    del Ad, Bd, C
    torch.cuda.empty_cache()


def test_misaligned_operand_is_rejected_without_launch(h):
    say("case misaligned A")
    dev = torch.device("cuda", 0)
    A = torch.ones((8, 24), dtype=torch.bfloat16, device=dev)
    C = torch.zeros((8, 8), dtype=torch.float32, device=dev)
    from dense_gemm_nt_amd import GemmError
    with pytest.raises(GemmError):
        h.run_raw(A.data_ptr() + 2, A.data_ptr(), C.data_ptr(), 8, 8, 16, 24, 24, 8, 0, 2, 0)


@pytest.mark.parametrize("M,N,K,splits", [(2100, 8300, 256, None), (4096, 4096, 512, 3),
                                          (8192, 8192, 192, None)])
def test_persistent_blocks_bitwise(M, N, K, splits):
    # persistent blocks (256 of them, several work units each, ragged edges, K
    # splits) run the same tile code: bitwise the grid launch's result, and the
    # oracle's on small integers
    say("case persistent M=%d N=%d K=%d splits=%s" % (M, N, K, splits))
    A, B = make_operands(M, N, K, "bf16", "int3", seed=M + K)
    hp = new_handle("256x256x64_w8_pp2", splits, persistent=True)
    Cp = run_gpu(hp, A, B, K, "bf16", "fp32")
    hp.close()
    hg = new_handle("256x256x64_w8_pp2", splits)
    Cg = run_gpu(hg, A, B, K, "bf16", "fp32")
    hg.close()
    assert np.array_equal(Cp, Cg)
    rows = [0, 255, 256, M - 1]
    Cr, _ = oracle.gemm_nt_rows(A, B, rows, K=K, in_dtype="bf16")
    assert np.array_equal(Cp[rows], Cr)
