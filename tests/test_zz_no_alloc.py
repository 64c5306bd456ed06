"""gemm_run_noalloc (the entry point for callers that cannot allocate) through the
C ABI, on the GPU: its output against gemm_run's on the same inputs, on two
calls in a row, the second with a smaller input; a shape whose default plan
needs more partials than the scratch holds; the same bits on a split plan that
fills the scratch and on small-M plans whose splits are reduced in the kernel;
and no device allocation once the scratch is loaded."""
import numpy as np
import pytest
import torch

import oracle
from gemm_inputs import make_operands
from tests.gpu_util import TORCH_DT, CODE, new_handle, run_gpu, say
from tests.tolerance import check

pytestmark = pytest.mark.gpu


def _noalloc(A_store, B_store, K, in_dt, out_dt):
    from dense_gemm_nt_amd import _lib
    M, lda = A_store.shape
    N, ldb = B_store.shape
    dev = torch.device("cuda", 0)
    Ad, Bd = A_store.to(dev), B_store.to(dev)
    Cd = torch.full((M, N), float("nan"), dtype=TORCH_DT[out_dt], device=dev)
    s = torch.cuda.current_stream(dev)
    st = _lib.lib().gemm_run_noalloc(Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), M, N, K, lda,
                                     ldb, N, CODE[in_dt], CODE[out_dt], s.cuda_stream)
    assert st == 0, _lib.STATUS.get(st, st)
    s.synchronize()
    return Cd.float().cpu().double().numpy()


def test_two_calls_in_a_row_match_gemm_run():
    h = new_handle()
    # first call: a split-K plan (the 256x128 tile, four splits, 32 MB of
    # partials in the scratch)
    M, N, K = 256, 8192, 8192
    say("case noalloc 1: M=%d N=%d K=%d bf16->bf16" % (M, N, K))
    A, B = make_operands(M, N, K, "bf16", "llm", seed=3)
    C1 = _noalloc(A, B, K, "bf16", "bf16")
    R1 = run_gpu(h, A, B, K, "bf16", "bf16")
    assert np.array_equal(C1, R1)            # same plan, same order: the same bits
    Cr, S = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    check(C1, Cr, S, "bf16", "noalloc 1")
    # second call, smaller: exact small integers with split-K partials
    M, N, K = 300, 280, 4104
    say("case noalloc 2: M=%d N=%d K=%d bf16->fp32 int3" % (M, N, K))
    A, B = make_operands(M, N, K, "bf16", "int3", seed=4, lda=K + 8)
    C2 = _noalloc(A, B, K, "bf16", "fp32")
    R2 = run_gpu(h, A, B, K, "bf16", "fp32")
    Cr, _ = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    assert np.array_equal(C2, R2) and np.array_equal(C2, Cr)
    h.close()


def test_plan_bounded_by_the_scratch():
    # stream-K here needs 128 MB of partials: the scratch takes the split plan
    # instead, whose result is within the bound of gemm_run's and the oracle's
    M, N, K = 3000, 3000, 5000
    say("case noalloc stream-K shape M=%d N=%d K=%d fp16->fp32" % (M, N, K))
    h = new_handle()
    A, B = make_operands(M, N, K, "fp16", "uniform", seed=0)
    C = _noalloc(A, B, K, "fp16", "fp32")
    R = run_gpu(h, A, B, K, "fp16", "fp32")
    Cr, S = oracle.gemm_nt(A, B, K=K, in_dtype="fp16")
    check(C, Cr, S, "fp32", "noalloc vs oracle")
    check(C, R, S, "fp32", "noalloc vs gemm_run")
    h.close()


def test_same_bits_on_a_split_plan_that_fills_the_scratch():
    # four K splits of 1024 x 4096 FP32 partials: the 64 MiB exactly; the same
    # plan as gemm_run's, so the same bits
    M, N, K = 1024, 4096, 8192
    say("case noalloc full scratch M=%d N=%d K=%d bf16->bf16" % (M, N, K))
    h = new_handle()
    A, B = make_operands(M, N, K, "bf16", "llm", seed=0)
    C = _noalloc(A, B, K, "bf16", "bf16")
    R = run_gpu(h, A, B, K, "bf16", "bf16")
    assert np.array_equal(C, R)
    h.close()


@pytest.mark.parametrize("M,N,K", [(1, 8192, 8192), (96, 8192, 8192), (20, 1000, 4104)])
def test_tile_kernel_in_kernel_reduction_matches_gemm_run(M, N, K):
    # small-M plans on the 32x128 and 128x128 tiles: K splits reduced in the
    # kernel through the scratch's slots and counters, in the rotated slab
    # order; the same plan as gemm_run's, so the same bits, and again on a
    # second call (the counters are back at zero)
    from dense_gemm_nt_amd import gemm_plan
    p = gemm_plan(M, N, K, 0, 0)
    assert p["splits"] > 1 and p["inreduce"] == 1, p
    say("case noalloc tile in-kernel M=%d N=%d K=%d %s splits=%d" % (M, N, K, p["name"], p["splits"]))
    h = new_handle()
    A, B = make_operands(M, N, K, "bf16", "llm", seed=M)
    R = run_gpu(h, A, B, K, "bf16", "bf16")
    for _ in range(2):
        assert np.array_equal(_noalloc(A, B, K, "bf16", "bf16"), R)
    h.close()


def test_no_device_allocation_after_the_first_call():
    M, N, K = 256, 10240, 8192
    say("case noalloc free memory unchanged M=%d N=%d K=%d" % (M, N, K))
    from dense_gemm_nt_amd import _lib
    dev = torch.device("cuda", 0)
    A, B = make_operands(M, N, K, "bf16", "llm", seed=9)
    Ad, Bd = A.to(dev), B.to(dev)
    Cd = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    s = torch.cuda.current_stream(dev)
    L = _lib.lib()

    def call():
        assert L.gemm_run_noalloc(Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), M, N, K, K, K, N,
                                  0, 0, s.cuda_stream) == 0

    call()                                   # loads the scratch on this device
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info(dev)
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info(dev)
    assert free1 == free0


def test_rejections_before_any_device_work():
    from dense_gemm_nt_amd import _lib
    L = _lib.lib()
    dev = torch.device("cuda", 0)
    A = torch.ones((8, 24), dtype=torch.bfloat16, device=dev)
    C = torch.zeros((8, 8), dtype=torch.float32, device=dev)
    assert L.gemm_run_noalloc(A.data_ptr() + 2, A.data_ptr(), C.data_ptr(), 8, 8, 16, 24, 24, 8,
                              0, 2, None) == 3                       # misaligned A
    assert L.gemm_run_noalloc(A.data_ptr(), A.data_ptr(), C.data_ptr(), 8, 8, 16, 8, 24, 8,
                              0, 2, None) == 1                       # lda < K
    assert L.gemm_run_noalloc(A.data_ptr(), A.data_ptr(), C.data_ptr(), 8, 8, 16, 24, 24, 8,
                              2, 2, None) == 2                       # FP32 inputs
    torch.cuda.synchronize()
    assert bool((C == 0).all())
