"""Host-side measurement and layout models pinned to the pages' printed tables."""
import os

import pytest

from dense_gemm_nt_amd import lds_model, roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_roofline_reproduces_page1_table():
    peak, bw, sms = 1500.0, 7.7, 148
    for ln in _rows("p1_roofline_table.csv"):
        name, M, N, K, fpb, bound, floor_us, kus, tf, tbs, ctas, wv = ln.split(",")
        M, N, K = int(M), int(N), int(K)
        r = roofline.roofline(M, N, K, 2, 2, peak_tflops=peak, hbm_tbs=bw)
        assert round(r.intensity) == int(fpb), name
        assert ("compute" if r.bound == "mfma" else "memory") == bound, name
        assert round(r.floor_us, 1) == float(floor_us), name
        kus = float(kus)
        assert round(roofline.flops(M, N, K) / kus / 1e6) == int(tf), name
        assert round(roofline.min_bytes(M, N, K, 2, 2) / kus / 1e6, 2) == float(tbs), name
        # 128x256 tiles counted as the page does (whole tiles)
        n_ctas = (M // 128) * (N // 256)
        assert n_ctas == int(ctas) and round(roofline.waves(n_ctas, sms), 2) == float(wv), name
    assert round(roofline.ridge(peak, bw)) == 195


def test_roofline_reproduces_other_page_figures():
    for ln in _rows("other_page_figures.txt"):
        parts = ln.split()
        if parts[0] == "p5_ceiling_tflops":
            M, N, K, ib, ob = map(int, parts[1:6])
            bw, want = float(parts[6]), float(parts[7])
            got = roofline.memory_ceiling_tflops(M, N, K, ib, ob, bw)
            assert abs(got - want) / want < 1e-3
        elif parts[0] == "p2_gflop":
            M, N, K = map(int, parts[1:4])
            assert round(roofline.flops(M, N, K) / 1e9, 1) == float(parts[4])


def test_mi355x_bounds_of_the_workloads():
    # square 4096^3 bf16 -> bf16 is compute bound; M=256 decode shapes are memory bound
    assert roofline.roofline(4096, 4096, 4096).bound == "mfma"
    for (M, N, K) in [(256, 28672, 8192), (256, 8192, 28672), (256, 10240, 8192), (256, 8192, 8192)]:
        assert roofline.roofline(M, N, K).bound == "hbm"
    assert abs(roofline.MI355X_NOMINAL_TFLOPS - 2516.58) < 0.01


def test_bank_model_reproduces_page1_table():
    rows = _rows("p1_swizzle_model.txt")
    for ln in rows:
        parts = ln.split()
        if parts[0] == "passes":
            tile_k, pitch, layout, want = int(parts[1]), int(parts[2]), parts[3], parts[4]
            f = (lambda a: a) if layout == "plain" else lds_model.page_swizzle
            got = [lds_model.group_passes([f(r * pitch + c * 16) for r in range(8)])
                   for c in range(pitch // 16)]
            assert got == [int(x) for x in want.split(",")], ln
        elif parts[0] == "perm":
            r = int(parts[1])
            got = [(lds_model.page_swizzle(r * 128 + c * 16) - r * 128) // 16 for c in range(8)]
            assert got == [int(x) for x in parts[2].split(",")]
    # the kernel's 128-byte key is the page's on rows 0..7
    for r in range(8):
        for c in range(8):
            assert lds_model.kernel_offset(r, c, 128) == lds_model.page_swizzle(r * 128 + c * 16)


@pytest.mark.parametrize("pitch", [128, 64])
def test_kernel_layouts_are_permutations_with_period_16(pitch):
    assert lds_model.load_map_is_permutation(pitch)
    assert lds_model.key_period_16(pitch)


def test_kernel_keys_serve_each_operand_read_group_in_one_pass():
    # 128-byte rows: one pass whether 8 lanes are served over 32 banks or 16
    # lanes over 64 banks; the page's key alone conflicts two-way at 64 banks
    assert lds_model.worst_read_passes(128, banks=32, lanes=8) == 1
    assert lds_model.worst_read_passes(128, banks=64, lanes=16) == 1
    page_key = lambda r: r & 7
    assert lds_model.worst_read_passes(128, banks=64, lanes=16, key=page_key) == 2
    # 64-byte rows (the four-wave tile's 32-deep stages): one pass at 64 banks
    assert lds_model.worst_read_passes(64, banks=64, lanes=16) == 1
    # unswizzled 64-byte rows: four rows share each bank group
    assert lds_model.worst_read_passes(64, banks=64, lanes=16, key=lambda r: 0) == 4
    # unswizzled 128-byte rows serialise fully at 32 banks
    assert lds_model.group_passes([r * 128 for r in range(8)]) == 8


def test_a_key_with_a_higher_row_bit_breaks_the_load_read_agreement():
    # ((r >> 1) ^ (r >> 3)) & 3 is conflict-free but depends on bit 4 of the
    # row: a load that computes it from the row within its 16-row group puts
    # rows 16..31 of each 32-row block where the operand read does not look
    bad = lambda r: ((r >> 1) ^ (r >> 3)) & 3
    assert lds_model.worst_read_passes(64, banks=64, lanes=16, key=bad) == 1
    assert not lds_model.key_period_16(64, key=bad)
