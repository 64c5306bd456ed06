"""The order in which tiles walk their k-slabs (GEMM_ROTATE), on the GPU,
through the C ABI.

A tile may start its k-slabs at a slab rotated per 256-column block, with a
partial last slab of K kept last: the same sum over the slabs in another order
("Matmul on sm_120", The tiled view: the tiled sum is the per-element sum in
another order).  So:

  * on small integers every partial sum is exact, and the natural order, the
    default rule (rotated when M <= 128) and rotation at every M give the
    oracle's bits, in every tile family, with and without K splits, with a
    partial last slab and with K % 8 != 0 (a slab visited twice or never
    would show here);
  * on random values each order is within the oracle's bound on every
    element;
  * the rule is a function of the problem: at M = 128 the default is the
    rotated order and at M = 129 the natural one, bit for bit, whatever tile
    the plan picks;
  * with rotation the two splits reduced in the kernel still equal the ordered
    second pass bitwise (the same slabs per split, in the same order).
"""
import numpy as np
import pytest

import oracle
from gemm_inputs import make_operands
from tests.gpu_util import compare_full, new_handle, run_gpu, say

pytestmark = pytest.mark.gpu

PP2, W4 = "256x256x64_w8_pp2", "256x128x64_w4_u8"
T128, T128_S2, T32, KMASK = "128x128x64_w8_s4", "128x128x64_w8_s2", "32x128x64_w4_s6", "128x128x64_w8_s4_kmask"

# (configuration, forced K splits, M, N, K): each family, a partial last slab
# (K % 64 != 0) on most, K splits whose ranges hold several slabs
CASES = [
    (T32, 3, 20, 1000, 4104),
    (T32, 1, 64, 520, 1544),
    (T128, 2, 100, 3000, 2056),
    (T128_S2, 1, 120, 2000, 1032),
    (KMASK, 1, 90, 700, 1001),
    (PP2, 2, 200, 1500, 4104),
    (PP2, 3, 300, 800, 3072),
    (W4, 3, 256, 1024, 8200),
]


@pytest.mark.parametrize("config,splits,M,N,K", CASES)
def test_every_order_small_integers_bitwise(config, splits, M, N, K):
    say("case slab order int3 %s splits=%d M=%d N=%d K=%d" % (config, splits, M, N, K))
    ld = -(-K // 8) * 8                       # row pitches a multiple of 8 elements
    A, B = make_operands(M, N, K, "bf16", "int3", seed=K + M, lda=ld, ldb=ld)
    Cr, _ = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    for rotate in (0, 1, 2):
        h = new_handle(config, splits, rotate=rotate)
        C = run_gpu(h, A, B, K, "bf16", "fp32")
        h.close()
        assert np.array_equal(C, Cr), rotate


@pytest.mark.parametrize("config,splits,M,N,K", CASES)
def test_rotated_order_random_every_element(config, splits, M, N, K):
    say("case slab order random %s splits=%d M=%d N=%d K=%d" % (config, splits, M, N, K))
    ld = -(-K // 8) * 8
    A, B = make_operands(M, N, K, "fp16", "uniform", seed=N, lda=ld, ldb=ld)
    for rotate in (0, 2):
        h = new_handle(config, splits, rotate=rotate)
        C = run_gpu(h, A, B, K, "fp16", "bf16")
        h.close()
        compare_full(C, A, B, K, "fp16", "bf16", "rotate=%d %s" % (rotate, config))


@pytest.mark.parametrize("M,same_as", [(1, 2), (64, 2), (128, 2), (129, 0), (256, 0)])
def test_default_rule_is_a_function_of_M(M, same_as):
    N, K = 2304, 4096
    say("case slab order rule M=%d (default = rotate %d)" % (M, same_as))
    A, B = make_operands(M, N, K, "bf16", "llm", seed=M)
    hd = new_handle()
    hs = new_handle(rotate=same_as)
    ho = new_handle(rotate=2 - same_as)
    Cd = run_gpu(hd, A, B, K, "bf16", "fp32")
    Cs = run_gpu(hs, A, B, K, "bf16", "fp32")
    Co = run_gpu(ho, A, B, K, "bf16", "fp32")
    for h in (hd, hs, ho):
        h.close()
    assert np.array_equal(Cd, Cs)
    # the other order sums differently somewhere (random values, K = 4096)
    assert not np.array_equal(Cd, Co)


@pytest.mark.parametrize("config", [PP2, W4])
def test_rotated_in_kernel_reduction_equals_second_pass_bitwise(config):
    M, N, K = 256, 4096, 8192
    say("case rotated in-kernel vs second pass %s M=%d N=%d K=%d" % (config, M, N, K))
    A, B = make_operands(M, N, K, "bf16", "llm", seed=3)
    h1 = new_handle(config, 2, inreduce=1, rotate=2)
    h0 = new_handle(config, 2, inreduce=0, rotate=2)
    C1 = run_gpu(h1, A, B, K, "bf16", "bf16")
    C0 = run_gpu(h0, A, B, K, "bf16", "bf16")
    h1.close()
    h0.close()
    assert np.array_equal(C1, C0)
