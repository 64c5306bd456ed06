"""The order in which tiles walk their k-slabs (GEMM_ROTATE), on the GPU,
through the C ABI.

The 32x128 and 128x128 tiles may start their k-slabs at a slab rotated per
256-column block, with a partial last slab of K kept last: the same sum over
the slabs in another order ("Matmul on sm_120", The tiled view: the tiled sum
is the per-element sum in another order).  The 256-row tiles always walk K
from the first slab.  So:

  * on small integers every partial sum is exact, and the natural order, the
    default rule (rotated when M <= 128) and rotation at every M give the
    oracle's bits, in every tile family, with and without K splits, with a
    partial last slab and with K % 8 != 0 (a slab visited twice or never
    would show here);
  * on random values each order is within the oracle's bound on every
    element;
  * the rule is a function of M: at M <= 128 the default plan is the rotated
    order and at M = 129 the natural one, bit for bit;
  * the 256-row tiles give the same bits under every mode.
"""
import numpy as np
import pytest

import oracle
from gemm_inputs import make_operands
from tests.gpu_util import compare_full, new_handle, run_gpu, say

pytestmark = pytest.mark.gpu

PP2, W4 = "256x256x64_w8_pp2", "256x128x64_w4_u8"
T128, T128_S2, T32, KMASK = "128x128x64_w8_s4", "128x128x64_w8_s2", "32x128x64_w4_s6", "128x128x64_w8_s4_kmask"

# (configuration, forced K splits, M, N, K): each tile family, a partial last
# slab (K % 64 != 0) on most, K splits whose ranges hold several slabs
CASES = [
    (T32, 3, 20, 1000, 4104),
    (T32, 1, 64, 520, 1544),
    (T128, 2, 100, 3000, 2056),
    (T128_S2, 1, 120, 2000, 1032),
    (KMASK, 1, 90, 700, 1001),
    (KMASK, 2, 300, 600, 3003),
    (PP2, 2, 200, 1500, 4104),
    (W4, 3, 256, 1024, 8200),
]


def _operands(M, N, K, dt, dist, seed):
    ld = -(-K // 8) * 8                       # row pitches a multiple of 8 elements
    return make_operands(M, N, K, dt, dist, seed=seed, lda=ld, ldb=ld)


@pytest.mark.parametrize("config,splits,M,N,K", CASES)
def test_every_order_small_integers_bitwise(config, splits, M, N, K):
    say("case slab order int3 %s splits=%d M=%d N=%d K=%d" % (config, splits, M, N, K))
    A, B = _operands(M, N, K, "bf16", "int3", K + M)
    Cr, _ = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    for rotate in (0, 1, 2):
        h = new_handle(config, splits, rotate=rotate)
        C = run_gpu(h, A, B, K, "bf16", "fp32")
        h.close()
        assert np.array_equal(C, Cr), rotate


@pytest.mark.parametrize("config,splits,M,N,K", CASES[:6])
def test_rotated_order_random_every_element(config, splits, M, N, K):
    say("case slab order random %s splits=%d M=%d N=%d K=%d" % (config, splits, M, N, K))
    A, B = _operands(M, N, K, "fp16", "uniform", N)
    out = {}
    for rotate in (0, 2):
        h = new_handle(config, splits, rotate=rotate)
        out[rotate] = run_gpu(h, A, B, K, "fp16", "fp32")
        h.close()
        compare_full(out[rotate], A, B, K, "fp16", "fp32", "rotate=%d %s" % (rotate, config))
    # three 256-column blocks or more and several slabs: the orders differ
    assert not np.array_equal(out[0], out[2])


@pytest.mark.parametrize("config,splits,M,N,K", CASES[6:])
def test_256_row_tiles_walk_k_in_order_under_every_mode(config, splits, M, N, K):
    say("case slab order ignored %s splits=%d M=%d N=%d K=%d" % (config, splits, M, N, K))
    A, B = _operands(M, N, K, "bf16", "llm", M)
    out = []
    for rotate in (0, 1, 2):
        h = new_handle(config, splits, rotate=rotate)
        out.append(run_gpu(h, A, B, K, "bf16", "fp32"))
        h.close()
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])


@pytest.mark.parametrize("M,config,rotated", [(1, None, True), (64, None, True), (128, None, True),
                                              (129, T128, False)])
def test_default_rule_is_a_function_of_M(M, config, rotated):
    # the default plans at M <= 128 are the 32x128 and 128x128 tiles; at
    # M = 129 the 128x128 tile is forced, where the rule turns rotation off
    N, K = 2304, 4096
    say("case slab order rule M=%d (rotated by default: %s)" % (M, rotated))
    A, B = make_operands(M, N, K, "bf16", "llm", seed=M)
    C = {}
    for rotate in (None, 0, 2):
        h = new_handle(config, rotate=rotate)
        C[rotate] = run_gpu(h, A, B, K, "bf16", "fp32")
        h.close()
    same, other = (2, 0) if rotated else (0, 2)
    assert np.array_equal(C[None], C[same])
    assert not np.array_equal(C[None], C[other])
