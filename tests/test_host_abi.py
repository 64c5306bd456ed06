"""The C-ABI library on the host: it loads, exports what the header declares, and
its argument checks and plans behave as documented.  No device work here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_nt.h")


@pytest.fixture(scope="module")
def g():
    import dense_gemm_nt_amd as g
    from dense_gemm_nt_amd import build
    if build.stale():
        build.build()
    return g


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(g):
    from dense_gemm_nt_amd import _lib
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    L = _lib.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(_lib.EXPORTS) == declared


def test_status_strings(g):
    assert g.gemm_status_string(0) == "GEMM_OK"
    assert g.gemm_status_string(3) == "GEMM_ERR_MISALIGNED"
    assert g.gemm_status_string(99) == "GEMM_ERR_UNKNOWN"


A16 = 0x10000          # a 16-byte aligned fake address (never dereferenced)


@pytest.mark.parametrize("args,want", [
    # (A, B, C, M, N, K, lda, ldb, ldc, in, out)
    ((A16, A16, A16, 4, 4, 8, 8, 8, 4, 0, 0), 0),
    ((A16, A16, A16, 4, 4, 8, 8, 8, 4, 1, 2), 0),
    ((A16, A16, A16, 4, 4, 8, 8, 8, 4, 2, 0), 2),     # fp32 inputs unsupported
    ((A16, A16, A16, 4, 4, 8, 8, 8, 4, 0, 7), 2),     # unknown output enum
    ((A16, A16, A16, -1, 4, 8, 8, 8, 4, 0, 0), 1),    # negative M
    ((A16, A16, A16, 4, 4, 8, 7, 8, 4, 0, 0), 1),     # lda < K
    ((A16, A16, A16, 4, 4, 8, 8, 8, 3, 0, 0), 1),     # ldc < N
    ((0, A16, A16, 4, 4, 8, 8, 8, 4, 0, 0), 1),       # null A
    ((A16, A16, 0, 4, 4, 8, 8, 8, 4, 0, 0), 1),       # null C
    ((A16 + 2, A16, A16, 4, 4, 8, 8, 8, 4, 0, 0), 3),  # A not 16-byte aligned
    ((A16, A16, A16, 4, 4, 8, 12, 8, 4, 0, 0), 3),    # lda not a multiple of 8
    ((A16, A16, A16 + 2, 4, 4, 8, 8, 8, 4, 0, 2), 3),  # fp32 C not 4-byte aligned
    ((A16, A16, A16 + 2, 4, 4, 8, 8, 8, 4, 0, 0), 0),  # bf16 C needs only 2 bytes
    ((0, 0, 0, 0, 4, 8, 8, 8, 4, 0, 0), 0),           # M = 0: nothing to do
    ((0, 0, A16, 4, 4, 0, 0, 0, 4, 0, 0), 0),         # K = 0: zeros, A/B unused
    ((A16, A16, A16, 4, 4, 8, 1 << 22, 8, 4, 0, 0), 2),  # lda beyond the limit
])
def test_validate(g, args, want):
    assert g.gemm_validate(*args) == want


def test_run_rejects_null_handle_before_any_device_work(g):
    from dense_gemm_nt_amd import _lib
    st = _lib.lib().gemm_run(None, A16, A16, A16, 4, 4, 8, 8, 8, 4, 0, 0, None)
    assert st == 1


def test_destroy_null_is_noop(g):
    from dense_gemm_nt_amd import _lib
    assert _lib.lib().gemm_destroy(None) == 0


def test_create_rejects_null_out(g):
    from dense_gemm_nt_amd import _lib
    assert _lib.lib().gemm_create(None) == 1


def test_create_rejects_unknown_forced_config_before_device_work(g, monkeypatch):
    # a measurement override naming no kernel must fail, not fall back silently
    import ctypes
    from dense_gemm_nt_amd import _lib
    monkeypatch.setenv("GEMM_CONFIG", "no_such_kernel")
    h = ctypes.c_void_p(12345)
    assert _lib.lib().gemm_create(ctypes.byref(h)) == 1
    assert h.value is None


LDS_BYTES = 160 * 1024


@pytest.mark.parametrize("M,N,K", [
    (512, 512, 512), (4096, 4096, 4096), (8192, 8192, 8192), (8192, 28672, 8192),
    (256, 28672, 8192), (256, 8192, 28672), (256, 10240, 8192), (256, 8192, 8192),
    (1000, 4097, 1536), (127, 28672, 8192), (3000, 3000, 5000), (1, 8192, 8192),
    (5, 7, 37), (33, 65, 1),
])
def test_plans_fit_the_machine(g, M, N, K):
    p = g.gemm_plan(M, N, K, 0, 0)
    bm, bn, bk = p["block_m"], p["block_n"], p["block_k"]
    assert 0 < p["lds_bytes"] <= LDS_BYTES
    assert p["lds_bytes"] >= 2 * (bm + bn) * bk * 2 or p["lds_bytes"] % (16 * 1024) == 0
    assert p["tiles"] == -(-M // bm) * -(-N // bn)
    k_tiles = -(-K // bk)
    if p["streamk"]:
        # every workgroup an equal run of the tiles * k_tiles units, one 256 KB
        # FP32 slot per tile segment it touches
        units = p["tiles"] * k_tiles
        G = min(256, units)
        assert p["splits"] == 1 and p["workgroups"] == G
        run = -(-units // G)
        assert p["workspace_bytes"] == G * ((run - 1) // k_tiles + 2) * 256 * 256 * 4
        assert p["workspace_bytes"] <= 128 << 20
        return
    assert p["workgroups"] == p["tiles"] * p["splits"]
    assert 1 <= p["splits"] <= max(1, k_tiles)
    if p["splits"] > 1 and p["inreduce"]:
        # reduced in the kernel: one BM x BN FP32 slot per tile and split
        assert p["workspace_bytes"] == p["tiles"] * p["splits"] * bm * bn * 4
        assert p["workspace_bytes"] <= 128 << 20
    elif p["splits"] > 1:
        assert p["workspace_bytes"] == p["splits"] * M * N * 4
        assert p["workspace_bytes"] <= 128 << 20
    else:
        assert p["workspace_bytes"] == 0
    if K % 8:
        assert p["name"].endswith("kmask")


def test_plan_regimes(g):
    # prefill / square: the big tile, one or more full waves of 256 CUs
    assert g.gemm_plan(4096, 4096, 4096)["tiles"] == 256
    assert g.gemm_plan(8192, 8192, 8192)["tiles"] == 1024
    # decode with few tiles splits K to cover the compute units
    p = g.gemm_plan(256, 8192, 8192)
    assert (p["splits"] > 1 or p["streamk"]) and p["workgroups"] >= 128
    # few big tiles with a long K: stream-K over all 256 compute units; with a
    # short K (runs under 32 k-slabs) or a well-filled split plan, not
    p = g.gemm_plan(3000, 3000, 5000)
    assert p["streamk"] == 1 and p["workgroups"] == 256 and p["splits"] == 1
    assert g.gemm_plan(3000, 3000, 1536)["streamk"] == 0
    assert g.gemm_plan(2304, 2304, 8192)["streamk"] == 0
    assert g.gemm_plan(3000, 3000, 3000)["streamk"] == 0
    assert g.gemm_plan(256, 28672, 8192)["streamk"] == 0
    assert g.gemm_plan(4096, 4096, 4096)["streamk"] == 0
    # mid-size M with a long K: the 256x256 tile with K splits fills the machine
    p = g.gemm_plan(512, 8192, 8192)
    assert p["name"] == "256x256x64_w8_pp2" and p["splits"] > 1 and p["workgroups"] >= 128
    # ... and with a short K the smaller tile keeps the compute units busy: two
    # blocks per compute unit when its tiles overflow one pass of the machine
    assert g.gemm_plan(1000, 4097, 1536)["name"] == "128x128x64_w8_s2"
    assert g.gemm_plan(1000, 4096, 1536)["name"] == "128x128x64_w8_s4"
    # the 32x128 tile where, in one pass with its own splits, it fills the
    # machine strictly better than the 128x128 tile (small squares, small
    # problems with short K); on a tie the 128x128 tile
    for M, N, K in ((178, 640, 2240), (74, 1408, 512), (618, 704, 3968)):
        assert g.gemm_plan(M, N, K)["name"] == "32x128x64_w4_s6", (M, N, K)
    assert g.gemm_plan(512, 512, 512)["name"] == "32x128x64_w4_s6"
    assert g.gemm_plan(1024, 1024, 1024)["name"] == "32x128x64_w4_s6"
    assert g.gemm_plan(640, 768, 8192)["name"] == "128x128x64_w8_s4"
    # small M: the 32x128 tile up to M = 64, with split counts whose K starts
    # are not a multiple of 4 KB apart (for M <= 32); the 128x128 tile from M = 96
    p = g.gemm_plan(1, 8192, 8192)
    assert p["name"] == "32x128x64_w4_s6" and p["splits"] == 3
    # for M <= 32 the K splits aim at about three quarters of the compute
    # units (rounded), not all of them
    for (M, N, K), sp in (((1, 4096, 16384), 6), ((1, 2048, 32768), 12), ((16, 4096, 4096), 6),
                          ((1, 16384, 8192), 3), ((1, 6144, 8192), 3)):
        p = g.gemm_plan(M, N, K)
        assert p["name"] == "32x128x64_w4_s6" and p["splits"] == sp, (M, N, K, p)
    # M = 64 (two tile rows sharing B) still fills every compute unit, and
    # reduces its splits in the kernel
    p = g.gemm_plan(64, 8192, 8192)
    assert p["name"] == "32x128x64_w4_s6" and p["splits"] == 2 and p["workgroups"] == 256
    assert p["inreduce"] == 1 and p["workspace_bytes"] == p["tiles"] * 2 * 32 * 128 * 4
    assert g.gemm_plan(96, 28672, 8192)["name"] == "128x128x64_w8_s4"
    # 32 < M <= 64: the 32x128 tile only while its tiles fit one pass
    assert g.gemm_plan(32, 28672, 8192)["name"] == "32x128x64_w4_s6"
    for M in (33, 40, 64):
        assert g.gemm_plan(M, 28672, 8192)["name"] == "128x128x64_w8_s4", M
        assert g.gemm_plan(M, 16384, 8192)["name"] == "32x128x64_w4_s6", M
    # two K splits on the 256-row tiles are reduced inside the kernel (one
    # 256 x 256 FP32 slot per split and tile); more splits take the second pass
    p = g.gemm_plan(256, 28672, 8192)
    assert p["splits"] == 2 and p["inreduce"] == 1
    assert p["workspace_bytes"] == p["tiles"] * 2 * p["block_m"] * p["block_n"] * 4
    # decode shapes the ping-pong tile would split more than four ways: the
    # 256x128 tile with half the splits, more than two of them reduced by a
    # second pass
    for N, K in ((10240, 8192), (8192, 8192), (8192, 28672)):
        p = g.gemm_plan(256, N, K)
        assert p["name"] == "256x128x64_w4_u8" and p["splits"] in (3, 4), p
        assert p["inreduce"] == 0 and p["workspace_bytes"] == p["splits"] * 256 * N * 4
    assert g.gemm_plan(256, 28672, 8192)["name"] == "256x256x64_w8_pp2"
    # 128 < M <= 256 with short K or few N tiles: the 256-row tiles only while
    # they fill the machine as well as the 128x128 tile
    for M, N, K in ((192, 4096, 4096), (256, 8192, 2048), (256, 2048, 8192), (200, 6144, 3072)):
        assert g.gemm_plan(M, N, K)["name"] == "128x128x64_w8_s4", (M, N, K)
    assert g.gemm_plan(256, 16384, 4096)["name"] == "256x128x64_w4_u8"
    # M > 256: the 128x128 tile where its tiles fit one pass and fill it at
    # least as well as the ping-pong tile
    for M, N, K in ((640, 2048, 8192), (768, 4096, 4096), (384, 8192, 4096)):
        assert g.gemm_plan(M, N, K)["name"] == "128x128x64_w8_s4", (M, N, K)
    assert g.gemm_plan(512, 16384, 2048)["name"] == "256x256x64_w8_pp2"
    # as full as the ping-pong tile, whose two splits would hold 32 slabs each
    assert g.gemm_plan(256, 28672, 4096)["name"] == "256x128x64_w4_u8"
    # more than two splits on the ping-pong tile take the second pass
    p = g.gemm_plan(512, 8192, 8192)
    assert p["name"] == "256x256x64_w8_pp2" and p["splits"] == 4 and p["inreduce"] == 0
    assert p["workspace_bytes"] == 4 * 512 * 8192 * 4
    assert g.gemm_plan(4096, 4096, 4096)["inreduce"] == 0
    # the 4 KB stride rule only moves a split count the fill rule chose: with
    # at least 256 tiles there is one split, and it stays one
    p = g.gemm_plan(1, 65536, 8192)
    assert p["name"] == "32x128x64_w4_s6" and p["tiles"] == 512 and p["splits"] == 1
    p = g.gemm_plan(32, 32768, 8192)
    assert p["tiles"] == 256 and p["splits"] == 1


def test_run_layout_rejects_null_handle_before_any_device_work(g):
    from dense_gemm_nt_amd import _lib
    st = _lib.lib().gemm_run_layout(None, 1, 1, A16, A16, A16, 4, 4, 8, 8, 8, 4, 0, 0, None, None)
    assert st == 1


def test_run_fp8_rejects_null_handle_and_scales_before_any_device_work(g):
    from dense_gemm_nt_amd import _lib
    L = _lib.lib()
    assert L.gemm_run_fp8(None, 3, 3, A16, A16, A16, 4, 4, 16, 16, 16, 4, 0, None, None, None) == 1


def test_run_grouped_rejects_null_handle_before_any_device_work(g):
    from dense_gemm_nt_amd import _lib
    assert _lib.lib().gemm_run_grouped(None, None, 0, 0, 0, None, None) == 1


def test_run_grouped_fp8_rejects_null_handle_before_any_device_work(g):
    from dense_gemm_nt_amd import _lib
    assert _lib.lib().gemm_run_grouped_fp8(None, 3, 3, None, 0, 0, 0, 1, None, None) == 1
