"""rocprofv3 over the configured workloads: one kernel-trace run and three counter
runs per workload, each a child process, then one short summary per workload.

    python -m dense_gemm_nt_amd.profile_workloads --out DIR [--workloads a,b,...]

Every run executes `python3 -m dense_gemm_nt_amd.profile_run --workload W`
(12 launches of the planned kernels on rotating inputs, then a 512 MiB device
copy) under rocprofv3, from /tmp with this repository on PYTHONPATH:

    trace:  rocprofv3 --kernel-trace --stats
    fetch:  rocprofv3 --pmc FETCH_SIZE
    write:  rocprofv3 --pmc WRITE_SIZE TCC_HIT_sum TCC_MISS_sum
    sq:     rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE
                            SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_WAIT_INST_LDS

(one counter group per run: FETCH_SIZE takes three of the four TCC counters a
run can hold, WRITE_SIZE two).  Each run has its own time limit; the first
failure ends the whole job.  Writes DIR/<workload>/... (raw CSV),
DIR/summaries/<plan>__<workload>.md and DIR/summaries/hbm_traffic.json (HBM
bytes per launch of the dominant kernel, calibrated by the copy).
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from dense_gemm_nt_amd import profile_summary as ps          # noqa: E402
from dense_gemm_nt_amd.profile_run import WORKLOADS          # noqa: E402

PASSES = [
    ("trace", ["--kernel-trace", "--stats"], 180),
    ("fetch", ["--pmc", "FETCH_SIZE"], 90),
    ("write", ["--pmc", "WRITE_SIZE", "TCC_HIT_sum", "TCC_MISS_sum"], 90),
    ("sq", ["--pmc", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
            "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS"], 90),
]
SKIP = 2          # warm-up launches left out of every average
COPY_MB = 512
XCDS, SIMDS = 8, 1024


def _cmd(out_dir, name, args, workload):
    return ["rocprofv3", *args, "-d", out_dir, "-o", name, "--output-format", "csv", "--",
            "python3", "-m", "dense_gemm_nt_amd.profile_run", "--workload", workload]


def _run(cmd, limit, log):
    env = dict(os.environ, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""),
               TMPDIR="/tmp")
    full = ["timeout", "-s", "KILL", str(limit), *cmd]
    print("run: " + " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(full, cwd="/tmp", env=env, stdout=f, stderr=subprocess.STDOUT)
    return r.returncode


def _find(out_dir, suffix):
    for dp, _, fs in os.walk(out_dir):
        for f in fs:
            if f.endswith(suffix):
                return os.path.join(dp, f)
    return None


def _plan(workload):
    """The library's plan for the workload, asked in a child process (this one
    never loads the HIP library, so it only ever starts children)."""
    M, N, K, ind, outd, _, _ = WORKLOADS[workload]
    code = {"bf16": 0, "fp16": 1, "fp32": 2}
    src = ("import json, dense_gemm_nt_amd as g; "
           "print(json.dumps(g.gemm_plan(%d, %d, %d, %d, %d)))" % (M, N, K, code[ind], code[outd]))
    env = dict(os.environ, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", src], env=env, capture_output=True, text=True,
                       check=True)
    return json.loads(r.stdout.strip().splitlines()[-1])


def _copy_reading(path, counter):
    """What `counter` read (KiB) for the calibration copy: the largest single
    dispatch of a copy kernel (the run's other copies move a few KiB)."""
    import csv
    best = 0.0
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if "copy" in (r.get("Kernel_Name") or "").lower() and r.get("Counter_Name") == counter:
                best = max(best, float(r.get("Counter_Value") or 0))
    return best


def _short_kernel(name):
    return name.replace("(gnt::KernelArgs)", "").replace("void ", "").replace(", int)", ")")


def summarize(workload, wdir, plan):
    M, N, K, ind, outd, dist, sets = WORKLOADS[workload]
    from dense_gemm_nt_amd import roofline
    ib, ob = roofline.DTYPE_BYTES[ind], roofline.DTYPE_BYTES[outd]
    alg = roofline.min_bytes(M, N, K, ib, ob)
    flops = roofline.flops(M, N, K)
    trace = ps.trace_groups(_find(os.path.join(wdir, "trace"), "kernel_trace.csv"))
    cnt = {}
    for p in ("fetch", "write", "sq"):
        for k, cs in ps.counters(_find(os.path.join(wdir, p), "counter_collection.csv"), SKIP).items():
            cnt.setdefault(k, {}).update(cs)
    scale = {}
    for cn, p in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        kib = _copy_reading(_find(os.path.join(wdir, p), "counter_collection.csv"), cn)
        if kib:
            scale[cn] = (COPY_MB << 20) / (kib * 1024.0)
    gemm = [k for k in cnt if "gnt::" in k]
    rows, total_us, traffic = [], 0.0, {"read": 0.0, "write": 0.0}
    dominant, dom_us = None, -1.0
    for k in gemm:
        ds = []
        for (n, _), v in trace.items():
            if n == k:
                ds += v[SKIP:] if len(v) > SKIP else v
        us = sum(ds) / len(ds) / 1e3 if ds else float("nan")
        cs = cnt[k]
        rd = cs["FETCH_SIZE"][0] * 1024.0 * scale.get("FETCH_SIZE", float("nan"))
        wr = cs["WRITE_SIZE"][0] * 1024.0 * scale.get("WRITE_SIZE", float("nan"))
        hit, miss = cs.get("TCC_HIT_sum", (0, 0))[0], cs.get("TCC_MISS_sum", (0, 0))[0]
        grbm = cs.get("GRBM_GUI_ACTIVE", (0, 0))[0] / XCDS
        mfma = cs.get("SQ_VALU_MFMA_BUSY_CYCLES", (0, 0))[0] / SIMDS
        rows.append({"kernel": _short_kernel(k), "us": us, "read": rd, "write": wr,
                     "l2_hit": hit / (hit + miss) if hit + miss else float("nan"),
                     "cycles": grbm, "mfma_busy": mfma / grbm if grbm else float("nan"),
                     "ghz": grbm / (us * 1e3) if us == us and us > 0 else float("nan"),
                     "lds_insts": cs.get("SQ_INSTS_LDS", (0, 0))[0],
                     "lds_conflicts": cs.get("SQ_LDS_BANK_CONFLICT", (0, 0))[0],
                     "lds_active": cs.get("SQ_LDS_IDX_ACTIVE", (0, 0))[0],
                     "dispatches": cs["FETCH_SIZE"][1]})
        total_us += us
        traffic["read"] += rd
        traffic["write"] += wr
        if us > dom_us:
            dominant, dom_us = k, us
    dom = next(r for r in rows if r["kernel"] == _short_kernel(dominant))
    mode = ("stream-K" if plan["streamk"] else
            "two K splits reduced in the kernel" if plan.get("inreduce") else
            "%d K splits + second-pass sum" % plan["splits"] if plan["splits"] > 1 else "one split")
    out = []
    out.append("# %s: %d x %d x %d, %s in, %s out (%s inputs), plan %s, %s, %d workgroups"
               % (workload, M, N, K, ind, outd, dist, plan["name"], mode, plan["workgroups"]))
    out.append("")
    out.append("Command (from the repository root on the GPU machine):")
    out.append("")
    out.append("    python -m dense_gemm_nt_amd.profile_workloads --out OUT --workloads %s" % workload)
    out.append("")
    out.append("which runs, from /tmp with the repository on PYTHONPATH:")
    out.append("")
    for name, args, _ in PASSES:
        out.append("    " + " ".join(_cmd("OUT/%s/%s" % (workload, name), name, args, workload)))
    out.append("")
    out.append("Device-source hash %s.  profile_run makes %d launches on %d rotating input sets; "
               "the first %d are left out of every figure.  Byte counters are calibrated "
               "by a %d MiB device copy (FETCH_SIZE x%.3f, WRITE_SIZE x%.3f)."
               % (ps.kernel_hash(), 12, sets, SKIP, COPY_MB, scale.get("FETCH_SIZE", float("nan")),
                  scale.get("WRITE_SIZE", float("nan"))))
    out.append("")
    out.append("| kernel | avg us (trace) | fabric read MB | fabric write MB | L2 hit | MFMA busy | "
               "clock GHz | LDS insts | LDS bank conflicts | dispatches |")
    out.append("|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        # (the clock only for MFMA kernels of more than 20 us: a short kernel's
        # GRBM count is mostly dispatch overhead)
        ghz = "%.2f" % r["ghz"] if r["mfma_busy"] > 0 and r["us"] > 20 else "-"
        out.append("| %s | %.2f | %.1f | %.1f | %.1f %% | %.1f %% | %s | %.4g | %.4g | %d |"
                   % (r["kernel"], r["us"], r["read"] / 1e6, r["write"] / 1e6, 100 * r["l2_hit"],
                      100 * r["mfma_busy"], ghz, r["lds_insts"], r["lds_conflicts"],
                      r["dispatches"]))
    out.append("")
    tb = traffic["read"] + traffic["write"]
    out.append("Per launch (all kernels): %.2f us, %.1f MB of fabric traffic for %.1f MB algorithmic "
               "(A and B read once, C written once): %.3f x.  Dominant kernel: %.1f MB "
               "(%.3f x).  %.1f TFLOP/s; %.0f GB/s of algorithmic bytes."
               % (total_us, tb / 1e6, alg / 1e6, tb / alg, (dom["read"] + dom["write"]) / 1e6,
                  (dom["read"] + dom["write"]) / alg, flops / (total_us * 1e-6) / 1e12,
                  alg / (total_us * 1e-6) / 1e9))
    out.append("")
    out.append("Fabric bytes are the L2's requests to memory (FETCH_SIZE, WRITE_SIZE): an upper "
               "bound on HBM traffic, since the memory-side cache may serve part of them.  "
               "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / %d SIMDs over GRBM_GUI_ACTIVE / %d XCDs; "
               "clock = those cycles over the traced duration." % (SIMDS, XCDS))
    entry = {"bytes_per_launch": dom["read"] + dom["write"], "read_bytes": dom["read"],
             "write_bytes": dom["write"], "fetch_calibration": scale.get("FETCH_SIZE"),
             "write_calibration": scale.get("WRITE_SIZE"), "kernel": dominant,
             "kernel_hash": ps.kernel_hash(),
             "plan": {"name": plan["name"], "splits": plan["splits"]},
             "launch_bytes_all_kernels": tb, "algorithmic_bytes": alg}
    return "\n".join(out) + "\n", entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--workloads", default=",".join(WORKLOADS))
    ap.add_argument("--summarize-only", action="store_true",
                    help="only rebuild the summaries from the CSV files under --out")
    args = ap.parse_args()
    out = os.path.abspath(args.out)
    names = [w for w in args.workloads.split(",") if w]
    for w in names:
        if w not in WORKLOADS:
            raise SystemExit("unknown workload %s" % w)
    sdir = os.path.join(out, "summaries")
    os.makedirs(sdir, exist_ok=True)
    tpath = os.path.join(sdir, "hbm_traffic.json")
    traffic = {}
    if os.path.exists(tpath):
        with open(tpath) as f:
            traffic = json.load(f)
    for w in names:
        wdir = os.path.join(out, w)
        if not args.summarize_only:
            for name, pargs, limit in PASSES:
                pdir = os.path.join(wdir, name)
                os.makedirs(pdir, exist_ok=True)
                t0 = time.time()
                rc = _run(_cmd(pdir, name, pargs, w), limit, os.path.join(pdir, "log.txt"))
                print("done: %s %s rc=%d %.1fs" % (w, name, rc, time.time() - t0), flush=True)
                if rc != 0:
                    raise SystemExit(rc)
        plan = _plan(w)
        text, entry = summarize(w, wdir, plan)
        M, N, K, ind, outd, _, _ = WORKLOADS[w]
        fname = "%s__%s.md" % (plan["name"], w)
        with open(os.path.join(sdir, fname), "w") as f:
            f.write(text)
        traffic["%dx%dx%d %s->%s" % (M, N, K, ind, outd)] = entry
        with open(tpath, "w") as f:
            json.dump(traffic, f, indent=1, sort_keys=True)
            f.write("\n")
        print("summary: %s" % fname, flush=True)


if __name__ == "__main__":
    main()
