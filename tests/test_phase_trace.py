"""The phase-trace analysis on synthetic records (no GPU): each quantity is the
difference of the right two events, per group, and the clock comes from the
reference clock."""
from dense_gemm_nt_amd import phase_trace as pt


def test_analysis_of_synthetic_records():
    # one block; group 0 waves: memory 1000, barrier 50, compute 1000, wait 10,
    # barrier 40; group 1 waves: compute 1100, barrier 60, memory 900, wait 20,
    # barrier 20 (both periods 2100 cycles); clock 2 GHz (2100 cycles per 1050 ns)
    blk = []
    for w in range(8):
        ev = []
        for i in range(pt.TN):
            t = 10_000 + 2100 * i
            r = 1_000_000 + 105 * i        # 100 MHz ticks: 1050 ns per slab
            if w < 4:
                ev.append([t, t + 1000, t + 1050, t + 2050, t + 2060, r])
            else:
                ev.append([t, t + 1100, t + 1160, t + 2060, t + 2080, r])
        blk.append(ev)
    tr = [blk] + [[[[0] * 6 for _ in range(pt.TN)] for _ in range(8)] for _ in range(pt.BLOCKS - 1)]
    rows, ghz = pt.analyse(tr)
    assert abs(ghz - 2.0) < 1e-9
    med = {k: pt._pct(v, 0.5) for k, v in rows.items()}
    assert med["period"] == 2100
    assert (med["g0_mem"], med["g0_bar1"], med["g0_comp"], med["g0_vmw"], med["g0_bar2"]) == (1000, 50, 1000, 10, 40)
    assert (med["g1_comp"], med["g1_bar1"], med["g1_mem"], med["g1_vmw"], med["g1_bar2"]) == (1100, 60, 900, 20, 20)
    # every wave contributes TN - 1 periods; empty blocks none
    assert len(rows["period"]) == 8 * (pt.TN - 1)
    assert len(rows["g0_mem"]) == 4 * (pt.TN - 1)


def test_layout_matches_the_kernel_header():
    src = open(pt.os.path.join(pt.PKG, "csrc", "gemm_nt_trace.hpp")).read()
    assert "TRACE_T0 = %d, TRACE_TN = %d, TRACE_REC = %d, TRACE_BLOCKS = %d" % (
        pt.T0, pt.TN, pt.REC, pt.BLOCKS) in src
