"""The rocprofv3 summariser on synthetic CSV files (no GPU, no profiler): byte
counters are calibrated by the largest copy dispatch only, warm-up dispatches are
left out, and MFMA busy / fabric bytes come out of the documented formulas."""
import csv
import os

from dense_gemm_nt_amd import profile_workloads as pw

GEMM = "void gnt::gemm_nt_pp2<0, 0, false, false, 0, false, 0>(gnt::KernelArgs)"
SUM = "void gnt::splitk_sum<0>(gnt::KernelArgs)"
COPY = "__amd_rocclr_copyBuffer"
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<unsigned char>>"


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def _trace_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Workgroup_Size_X", "Grid_Size_X", "Start_Timestamp",
                    "End_Timestamp"])
        for r in rows:
            w.writerow(r)


def _dispatches(counter, gemm_val, sum_val, copy_big, copy_small, fill):
    rows, d = [], 1
    rows.append((d, COPY, counter, copy_small)); d += 1        # small input copies
    rows.append((d, COPY, counter, copy_small)); d += 1
    for i in range(12):
        # the two warm-up launches read ten times more: they must be skipped
        rows.append((d, GEMM, counter, gemm_val * (10 if i < 2 else 1))); d += 1
        rows.append((d, SUM, counter, sum_val)); d += 1
    rows.append((d, FILL, counter, fill)); d += 1
    rows.append((d, COPY, counter, copy_big)); d += 1
    return rows


def test_summary_calibration_and_formulas(tmp_path):
    w = "decode_mlp_down"                     # 256 x 8192 x 28672, bf16 -> bf16
    wdir = str(tmp_path / w)
    big = 512 * 1024                          # KiB a 512 MiB copy should move
    # FETCH_SIZE reads half of what the copy moves (calibration x2); the fill
    # reads nothing and must not be taken for the calibration
    _counter_csv(os.path.join(wdir, "fetch", "fetch_counter_collection.csv"),
                 _dispatches("FETCH_SIZE", 1000.0, 100.0, big / 2, 12.0, 20.0))
    wr = _dispatches("WRITE_SIZE", 300.0, 30.0, big, 12.0, big)
    wr += [(r[0], r[1], "TCC_HIT_sum", 3.0) for r in wr] + [(r[0], r[1], "TCC_MISS_sum", 1.0) for r in wr]
    _counter_csv(os.path.join(wdir, "write", "write_counter_collection.csv"), wr)
    sq = []
    for r in _dispatches("GRBM_GUI_ACTIVE", 8 * 2000.0, 8 * 100.0, 1.0, 1.0, 1.0):
        sq.append(r)
        sq.append((r[0], r[1], "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500.0 if r[1] == GEMM else 0.0))
    _counter_csv(os.path.join(wdir, "sq", "sq_counter_collection.csv"), sq)
    tr = []
    t = 0
    for i in range(12):
        tr.append((GEMM, 512, 512 * 256, t, t + (50000 if i < 2 else 1000)))   # 1 us after warm-up
        t += 100000
        tr.append((SUM, 256, 256 * 64, t, t + 500))
        t += 100000
    _trace_csv(os.path.join(wdir, "trace", "trace_kernel_trace.csv"), tr)

    plan = {"name": "256x256x64_w8_pp2", "splits": 8, "streamk": 0, "inreduce": 0,
            "workgroups": 256}
    text, entry = pw.summarize(w, wdir, plan)
    assert entry["fetch_calibration"] == 2.0 and entry["write_calibration"] == 1.0
    assert entry["read_bytes"] == 1000.0 * 1024 * 2          # warm-ups left out
    assert entry["write_bytes"] == 300.0 * 1024
    assert entry["bytes_per_launch"] == entry["read_bytes"] + entry["write_bytes"]
    assert entry["kernel"] == GEMM
    assert entry["launch_bytes_all_kernels"] == (1000.0 * 2 + 300.0 + 100.0 * 2 + 30.0) * 1024
    assert entry["algorithmic_bytes"] == 2 * (256 * 28672 + 8192 * 28672) + 2 * 256 * 8192
    assert entry["plan"] == {"name": "256x256x64_w8_pp2", "splits": 8}
    # one GEMM row: 1 us, MFMA busy 500 / 2000 cycles, L2 hit 3 / 4, clock 2000 cycles / 1 us
    row = [ln for ln in text.splitlines() if ln.startswith("| gnt::gemm_nt_pp2")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "1.00"
    assert cells[4] == "75.0 %" and cells[5] == "25.0 %"
    assert cells[6] == "-"                                    # under 20 us: no clock
    assert "8 K splits + second-pass sum" in text
    assert "python -m dense_gemm_nt_amd.profile_workloads --out OUT --workloads %s" % w in text
