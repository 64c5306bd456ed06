"""Every output element against the oracle on seeded shapes drawn from each
regime of the planner, through the default plan (no forced configuration):
small M with stride-aware K splits, small squares on the 32x128 tile, the
128x128 tiles (one or two blocks per compute unit), the 256x256 ping-pong tile
with and without K splits.  The shapes are drawn once from a fixed seed, so a
failure names a shape that reproduces.  Bound: tests/tolerance.py.
"""
import numpy as np
import pytest

from dense_gemm_nt_amd import gemm_plan, _lib
from gemm_inputs import make_operands
from tests.gpu_util import compare_full, new_handle, run_gpu, say

pytestmark = pytest.mark.gpu

CODE = {"bf16": _lib.GEMM_BF16, "fp16": _lib.GEMM_FP16, "fp32": _lib.GEMM_FP32}


def _shapes():
    rng = np.random.default_rng(20261202)
    regimes = [
        # (M range, N range, K range): small M with long K (K splits); small
        # squares; 96 < M <= 128 (128x128 tile with K splits); 128x128 tiles
        # just past one pass of the machine (two blocks per compute unit);
        # 128 < M <= 256 with few N tiles (128x128 tile, K splits); mid
        # squares; 128 < M <= 256 with many N tiles (ping-pong tile, K splits)
        ((1, 64), (100, 1200), (1024, 4096)),
        ((257, 700), (257, 700), (64, 1100)),
        ((97, 128), (2000, 6000), (512, 2048)),
        ((990, 1020), (4100, 4300), (256, 512)),
        ((129, 256), (300, 1500), (2048, 6000)),
        ((1500, 2100), (1500, 2100), (256, 768)),
        # decode-like with many N tiles: the ping-pong tile with two K splits
        ((129, 256), (14000, 18000), (6000, 8200)),
    ]
    out = []
    for (m0, m1), (n0, n1), (k0, k1) in regimes:
        for _ in range(3):
            M = int(rng.integers(m0, m1 + 1))
            N = int(rng.integers(n0, n1 + 1))
            K = int(rng.integers(k0 // 8, k1 // 8 + 1)) * 8
            out.append((M, N, K))
    return out


SHAPES = _shapes()
DTS = [("bf16", "bf16"), ("fp16", "fp32"), ("bf16", "fp32"), ("fp16", "fp16")]


@pytest.mark.parametrize("i", range(len(SHAPES)), ids=["%dx%dx%d" % s for s in SHAPES])
def test_default_plan_every_element(i):
    M, N, K = SHAPES[i]
    ind, outd = DTS[i % len(DTS)]
    p = gemm_plan(M, N, K, CODE[ind], CODE[outd])
    say("case plan M=%d N=%d K=%d %s->%s %s splits=%d streamk=%d" % (
        M, N, K, ind, outd, p["name"], p["splits"], p["streamk"]))
    h = new_handle()
    A, B = make_operands(M, N, K, ind, "uniform", seed=i)
    C = run_gpu(h, A, B, K, ind, outd, ldc=N + (i % 3))
    err, worst = compare_full(C, A, B, K, ind, outd, "M=%d N=%d K=%d" % (M, N, K))
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))
    h.close()


def test_the_draw_reaches_each_tile_family():
    names = {gemm_plan(M, N, K)["name"] for M, N, K in SHAPES}
    assert {"32x128x64_w4_s6", "128x128x64_w8_s4", "128x128x64_w8_s2", "256x256x64_w8_pp2"} <= names, names


def test_plan_cache_over_many_shapes():
    # one handle through all the planner regimes above (more shapes than its
    # plan cache holds), then the first shapes again: every call gives the bits
    # a fresh handle gives (same plan, same summation order)
    h = new_handle()
    order = list(range(len(SHAPES))) + [0, 1, 2, len(SHAPES) - 1]
    for n, i in enumerate(order):
        M, N, K = SHAPES[i]
        say("case plan cache call %d: M=%d N=%d K=%d" % (n, M, N, K))
        A, B = make_operands(M, N, K, "bf16", "uniform", seed=100 + n)
        C = run_gpu(h, A, B, K, "bf16", "fp32")
        h2 = new_handle()
        R = run_gpu(h2, A, B, K, "bf16", "fp32")
        h2.close()
        assert np.array_equal(C, R), (M, N, K)
    h.close()


@pytest.mark.parametrize("M,N,K,splits", [(1, 4096, 16384, 6), (1, 2048, 32768, 12), (16, 4096, 4096, 6),
                                          (7, 6144, 8192, 3)])
def test_small_m_split_counts_every_element(M, N, K, splits):
    # M <= 32: the K splits aim at three quarters of the compute units; every
    # element of those split counts against the oracle, partials summed by
    # the second pass
    p = gemm_plan(M, N, K, CODE["bf16"], CODE["bf16"])
    assert p["name"] == "32x128x64_w4_s6" and p["splits"] == splits, p
    say("case small-M plan M=%d N=%d K=%d splits=%d" % (M, N, K, splits))
    h = new_handle()
    A, B = make_operands(M, N, K, "bf16", "llm", seed=M + splits)
    C = run_gpu(h, A, B, K, "bf16", "bf16")
    err, worst = compare_full(C, A, B, K, "bf16", "bf16", "M=%d N=%d K=%d" % (M, N, K))
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))
    h.close()


@pytest.mark.parametrize("M,N,K", [(1, 128, 1 << 20), (5, 260, (1 << 18) + 8)])
def test_longest_k_every_element(M, N, K):
    # one or three tiles with a K of a million: the split rule's largest
    # counts (191 and 64 splits of the 32-row tile), the ordered second pass
    # over all of them, and a ragged last split
    p = gemm_plan(M, N, K, CODE["bf16"], CODE["fp32"])
    say("case longest K M=%d N=%d K=%d %s splits=%d" % (M, N, K, p["name"], p["splits"]))
    assert p["splits"] >= 64, p
    h = new_handle()
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=K % 97)
    C = run_gpu(h, A, B, K, "bf16", "fp32")
    err, worst = compare_full(C, A, B, K, "bf16", "fp32", "M=%d N=%d K=%d" % (M, N, K))
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))
    h.close()


# The tile choices made by how full a pass each family would be: the 128x128
# tile for 32 < M <= 64 past one pass of 32-row tiles, for 128 < M <= 256
# with short K or few N tiles, and above M = 256 where its tiles fit one
# pass; the four-wave tile over the ping-pong one.  Every element against
# the oracle, through the default plan.
FILL_CASES = [((40, 20480, 4096), "128x128x64_w8_s4"), ((200, 6144, 3072), "128x128x64_w8_s4"),
              ((256, 2048, 8192), "128x128x64_w8_s4"), ((640, 2048, 8192), "128x128x64_w8_s4"),
              ((384, 4096, 2048), "128x128x64_w8_s4"), ((256, 16384, 4096), "256x128x64_w4_u8"),
              ((256, 28672, 4096), "256x128x64_w4_u8"),
              # above M = 64, the 32x128 tile where its tiles fill one pass
              # strictly better (M not a multiple of 32 on all three, N not a
              # multiple of 128 on the last)
              ((178, 640, 2240), "32x128x64_w4_s6"), ((74, 1408, 512), "32x128x64_w4_s6"),
              ((618, 704, 3968), "32x128x64_w4_s6")]


@pytest.mark.parametrize("shape,name", FILL_CASES, ids=["%dx%dx%d" % s for s, _ in FILL_CASES])
def test_fill_rule_plans_every_element(shape, name):
    M, N, K = shape
    p = gemm_plan(M, N, K, CODE["bf16"], CODE["bf16"])
    assert p["name"] == name, p
    say("case fill-rule plan M=%d N=%d K=%d %s splits=%d" % (M, N, K, p["name"], p["splits"]))
    h = new_handle()
    A, B = make_operands(M, N, K, "bf16", "llm", seed=M + N)
    C = run_gpu(h, A, B, K, "bf16", "bf16")
    compare_full(C, A, B, K, "bf16", "bf16", "fill rule M=%d N=%d K=%d" % (M, N, K))
    h.close()
