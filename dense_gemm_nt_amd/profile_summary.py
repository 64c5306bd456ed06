"""Summarise rocprofv3 CSV output into the short text kept under profiles/.

    python -m dense_gemm_nt_amd.profile_summary --stats DIR/run_kernel_stats.csv
    python -m dense_gemm_nt_amd.profile_summary --trace DIR/run_kernel_trace.csv
    python -m dense_gemm_nt_amd.profile_summary --counters DIR/fetch_counter_collection.csv \
        [--copy-mb 512] [--skip 2]
    python -m dense_gemm_nt_amd.profile_summary --traffic FETCH.csv WRITE.csv \
        --key "4096^3 bf16->bf16" --plan 256x256x64_w8_pp2:1 --update profiles/hbm_traffic.json

Counter mode averages each counter over the GEMM dispatches (after `--skip`
warm-up launches) and, for FETCH_SIZE / WRITE_SIZE (KiB per dispatch), scales the
GEMM reading by the bytes a plain copy of --copy-mb MiB must move divided by what
the same counter read for that copy.
"""
from __future__ import annotations

import argparse
import csv
import json
from collections import OrderedDict, defaultdict


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name):
    return name if len(name) < 110 else name[:107] + "..."


def stats(path):
    out = []
    for r in _rows(path):
        out.append((r.get("Name") or r.get("KernelName") or "?", int(r.get("Calls", 0)),
                    float(r.get("AverageNs", 0)), float(r.get("MinNs", 0)), float(r.get("MaxNs", 0)),
                    float(r.get("Percentage", 0))))
    return out


def trace_groups(path):
    """Per-dispatch kernel trace grouped by (kernel, workgroups): one workload each
    when one kernel serves several grid shapes.  Durations in ns."""
    groups = OrderedDict()
    for r in _rows(path):
        name = r.get("Kernel_Name") or "?"
        wg = int(r.get("Workgroup_Size_X") or 1) * int(r.get("Workgroup_Size_Y") or 1) * \
            int(r.get("Workgroup_Size_Z") or 1)
        grid = int(r.get("Grid_Size_X") or 0) * int(r.get("Grid_Size_Y") or 1) * \
            int(r.get("Grid_Size_Z") or 1)
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        groups.setdefault((name, grid // max(wg, 1)), []).append(d)
    return groups


def leading_run(path, name, workgroups):
    """Durations (ns) of the first unbroken run of dispatches of one kernel at one
    grid size, in dispatch order: the workload a bench step times first, before
    later workloads launch the same kernel at the same grid."""
    rows = []
    for r in _rows(path):
        wg = int(r.get("Workgroup_Size_X") or 1) * int(r.get("Workgroup_Size_Y") or 1) * \
            int(r.get("Workgroup_Size_Z") or 1)
        grid = int(r.get("Grid_Size_X") or 0) * int(r.get("Grid_Size_Y") or 1) * \
            int(r.get("Grid_Size_Z") or 1)
        rows.append((int(r["Start_Timestamp"]), r.get("Kernel_Name") or "?", grid // max(wg, 1),
                     int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    run, started = [], False
    for _, n, g, d in rows:
        if n == name and g == workgroups:
            run.append(d)
            started = True
        elif started and "copyBuffer" not in n and "elementwise" not in n:
            break
    return run


def counters(path, skip):
    per = defaultdict(lambda: defaultdict(list))   # kernel -> counter -> values in dispatch order
    order = OrderedDict()
    for r in _rows(path):
        name = r.get("Kernel_Name") or r.get("Kernel-Name") or "?"
        cn = r.get("Counter_Name") or r.get("Counter-Name")
        cv = float(r.get("Counter_Value") or r.get("Counter-Value") or 0)
        did = int(r.get("Dispatch_Id") or r.get("Dispatch-Id") or 0)
        per[name][cn].append((did, cv))
        order[name] = True
    res = {}
    for name in order:
        res[name] = {}
        for cn, vals in per[name].items():
            vals.sort()
            v = [x for _, x in vals]
            if "gnt::" in name and len(v) > skip:
                v = v[skip:]
            res[name][cn] = (sum(v) / len(v), len(v))
    return res


def kernel_hash():
    """Same hash bench.py compares against: every source file of the library
    (all kernels, their launch tables and the host planner) as it is now; the
    plan is recorded beside the counters too."""
    import hashlib
    import os
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(root)):
        if f.endswith((".hip", ".hpp", ".h")):
            h.update(f.encode() + b"\0")
            with open(os.path.join(root, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def traffic(fetch_csv, write_csv, copy_mb, skip):
    """Calibrated HBM-side bytes per GEMM dispatch: (read, write, kernel name)."""
    out = {}
    for cn, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        res = counters(path, skip)
        scale = None
        for name, cs in res.items():
            if ("copy" in name.lower()) and cn in cs and cs[cn][0] > 0:
                scale = (copy_mb << 20) / (cs[cn][0] * 1024.0)
        if scale is None:
            raise SystemExit("no copy kernel found in %s for calibration" % path)
        gemm = [(n, cs[cn][0]) for n, cs in res.items() if "gemm_nt" in n and cn in cs]
        if not gemm:
            raise SystemExit("no GEMM kernel in %s" % path)
        # the dominant GEMM kernel (largest counter value) of the run
        name, kib = max(gemm, key=lambda t: t[1])
        out[cn] = (kib * 1024.0 * scale, scale, name)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats")
    ap.add_argument("--trace")
    ap.add_argument("--counters")
    ap.add_argument("--copy-mb", type=int, default=512)
    ap.add_argument("--skip", type=int, default=2)
    ap.add_argument("--json", action="store_true")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--key", help="workload key for --traffic")
    ap.add_argument("--update", help="JSON file to add the --traffic result to")
    ap.add_argument("--plan", help="for --traffic: the plan the counters ran, NAME:SPLITS")
    args = ap.parse_args()
    if args.traffic:
        t = traffic(args.traffic[0], args.traffic[1], args.copy_mb, args.skip)
        entry = {"bytes_per_launch": t["FETCH_SIZE"][0] + t["WRITE_SIZE"][0],
                 "read_bytes": t["FETCH_SIZE"][0], "write_bytes": t["WRITE_SIZE"][0],
                 "fetch_calibration": t["FETCH_SIZE"][1], "write_calibration": t["WRITE_SIZE"][1],
                 "kernel": t["FETCH_SIZE"][2], "kernel_hash": kernel_hash()}
        if args.plan:
            name, splits = args.plan.rsplit(":", 1)
            entry["plan"] = {"name": name, "splits": int(splits)}
        print(json.dumps({args.key: entry}, indent=1))
        if args.update:
            import os
            d = {}
            if os.path.exists(args.update):
                with open(args.update) as f:
                    d = json.load(f)
            d[args.key] = entry
            with open(args.update, "w") as f:
                json.dump(d, f, indent=1, sort_keys=True)
                f.write("\n")
        return
    if args.stats:
        print("| kernel | calls | avg us | min us | max us | % time |")
        print("|---|---|---|---|---|---|")
        for n, c, a, lo, hi, pct in stats(args.stats):
            print("| %s | %d | %.2f | %.2f | %.2f | %.1f |" % (_short(n), c, a / 1e3, lo / 1e3, hi / 1e3, pct))
    if args.trace:
        print("| kernel | workgroups | calls | avg us | min us | max us |")
        print("|---|---|---|---|---|---|")
        for (n, wgs), ds in trace_groups(args.trace).items():
            print("| %s | %d | %d | %.2f | %.2f | %.2f |" % (_short(n), wgs, len(ds), sum(ds) / len(ds) / 1e3,
                                                          min(ds) / 1e3, max(ds) / 1e3))
    if args.counters:
        res = counters(args.counters, args.skip)
        copy_bytes = args.copy_mb << 20
        scale = {}
        for name, cs in res.items():
            if "copy" in name.lower() or "elementwise" in name.lower():
                for cn in ("FETCH_SIZE", "WRITE_SIZE"):
                    if cn in cs and cs[cn][0] > 0:
                        scale[cn] = copy_bytes / (cs[cn][0] * 1024.0)
        summary = {}
        for name, cs in res.items():
            for cn, (avg, n) in sorted(cs.items()):
                line = {"avg": avg, "dispatches": n}
                if cn in ("FETCH_SIZE", "WRITE_SIZE"):
                    line["bytes_raw"] = avg * 1024.0
                    if cn in scale:
                        line["calibration"] = scale[cn]
                        line["bytes_calibrated"] = avg * 1024.0 * scale[cn]
                summary.setdefault(_short(name), {})[cn] = line
        if args.json:
            print(json.dumps(summary, indent=1))
        else:
            for name, cs in summary.items():
                print("kernel: %s" % name)
                for cn, line in cs.items():
                    extra = ""
                    if "bytes_calibrated" in line:
                        extra = "  -> %.1f MB (x%.3f from the copy calibration)" % (
                            line["bytes_calibrated"] / 1e6, line["calibration"])
                    print("  %-28s avg %.6g over %d dispatches%s" % (cn, line["avg"], line["dispatches"], extra))


if __name__ == "__main__":
    main()
