#!/usr/bin/env python3
"""Throughput of the MI355X NT GEMM on its headline workload.

One step = one call of the library (C = A . B^T) on one set of synthetic inputs
that are already resident in HBM.  Input sets rotate so the 256 MB last-level
cache cannot hold them across steps (cold-cache numbers).  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--quick]
    python bench.py --all-configs [--config NAME ...]

Primary workload: M = N = K = 4096, BF16 inputs uniform on [-1, 1), FP32
accumulation, BF16 output.  A second line item in the same JSON object reports
the decode-regime shape M = 256, N = 28672, K = 8192 (A ~ N(0,1), B ~ N(0, 0.02^2)),
an "extensions" list times the other forms of the product (operand
layouts, fused epilogue, FP8 with scales, grouped launch) on their workloads,
and a "configs" list gives every configured workload (CONFIGS below): median,
p10 and p90 of 50 launches each between HIP events, its roofline fraction and
an oracle spot check.  --all-configs prints only those, one JSON line each.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2500.0     # MI355X dense BF16/FP16 MFMA, published
HBM_TBS = 8.0            # MI355X HBM3E, published
def kernel_hash() -> str:
    from dense_gemm_nt_amd.profile_summary import kernel_hash as kh
    return kh()


def traffic_for(workload_key: str, plan: dict):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the kernel as it is now (same device-source hash) and with the plan
    this run uses (same kernel configuration and K splits); else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(workload_key)
    if not e or e.get("kernel_hash") != kernel_hash():
        return None
    rec = e.get("plan")
    if not rec or rec.get("name") != plan["name"] or rec.get("splits") != plan["splits"]:
        return None
    return e.get("bytes_per_launch")


def time_gemm(g, shapes, steps, warmup, sets, in_dt, out_dt, dist):
    import torch
    from gemm_inputs import make_operands
    M, N, K = shapes
    dev = torch.device("cuda", 0)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    code = {"bf16": 0, "fp16": 1, "fp32": 2}
    bufs = []
    for i in range(sets):
        A, B = make_operands(M, N, K, in_dt, dist, seed=i)
        bufs.append((A.to(dev), B.to(dev), torch.empty((M, N), dtype=tdt[out_dt], device=dev)))
        del A, B
    h = g.Gemm()
    stream = torch.cuda.Stream(device=dev)
    sp = stream.cuda_stream

    def launch(i):
        A, B, C = bufs[i % sets]
        h.run_raw(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, K, K, N,
                  code[in_dt], code[out_dt], sp)

    with torch.cuda.stream(stream):
        # settle: clocks, TLBs and caches reach steady state before the counted
        # warm-up steps (at least 0.3 s of back-to-back launches)
        settle, t_settle = 0, time.perf_counter()
        while time.perf_counter() - t_settle < 0.3:
            for _ in range(10):
                launch(settle)
                settle += 1
            torch.cuda.synchronize()
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            launch(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / steps
    event_ms = ev0.elapsed_time(ev1) / steps
    # the output of the last step, for a parity spot check
    last = (steps - 1) % sets
    h.close()
    return wall_ms, event_ms, bufs, last, settle


def spot_check(bufs, idx, shapes, in_dt, out_dt, dist, seed=None):
    """Oracle on two rows and 2000 points of the output bufs[idx][2], made from
    the input set drawn with `seed` (default: idx)."""
    import numpy as np
    import oracle
    from gemm_inputs import make_operands
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from tests.tolerance import check
    M, N, K = shapes
    A, B = make_operands(M, N, K, in_dt, dist, seed=idx if seed is None else seed)
    C = bufs[idx][2].float().cpu().double().numpy()
    rows = [0, M - 1]
    Cr, S = oracle.gemm_nt_rows(A, B, rows, K=K, in_dtype=in_dt)
    e1, w1 = check(C[rows], Cr, S, out_dt, "bench rows")
    rng = np.random.default_rng(1)
    ii, jj = rng.integers(0, M, 2000), rng.integers(0, N, 2000)
    Cp, Sp = oracle.gemm_nt_points(A, B, ii, jj, K=K, in_dtype=in_dt)
    e2, w2 = check(C[ii, jj], Cp, Sp, out_dt, "bench points")
    return max(w1, w2)


def _event_time(launch, iters, warmup, stream, settle_s=0.3):
    """Average duration of `launch()` over `iters` back-to-back calls on `stream`
    (HIP events on that stream), after a settle phase (launches for `settle_s`
    seconds, as before the primary timing: a GPU that sat idle runs its first
    launches at a lower clock) and `warmup` calls."""
    import torch
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < settle_s:
            launch()
            n += 1
            if n % 10 == 0:
                torch.cuda.synchronize()
        for _ in range(warmup):
            launch()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e-3      # seconds


def extensions(g, iters=30, warmup=10):
    """The other forms of the product on their own workloads: operand layouts,
    the fused epilogue, FP8 with scales and the grouped launch.  Each is timed
    with HIP events on its stream and spot-checked against the oracle."""
    import numpy as np
    import torch
    import oracle
    from oracle import epilogue as oepi
    from oracle import fp8 as ofp8
    from gemm_inputs import make_fp8_operands, make_operands, make_stored
    from tests.tolerance import check, check_epilogue
    from dense_gemm_nt_amd import _lib
    dev = torch.device("cuda", 0)
    stream = torch.cuda.Stream(device=dev)
    sp = stream.cuda_stream
    h = g.Gemm()
    rng = np.random.default_rng(7)
    res = []
    M = N = K = 4096
    flops = 2.0 * M * N * K
    ii, jj = rng.integers(0, M, 1000), rng.integers(0, N, 1000)

    # NN: row-major A times row-major B [K, N] (B stored N-major)
    Xa, Xb = make_stored(M, N, K, "k", "mn", "bf16", "uniform", seed=0)
    Ad, Bd = Xa.to(dev), Xb.to(dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t = _event_time(lambda: h.run_raw_layout(0, 1, Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), M,
                                             N, K, K, N, N, 0, 0, None, sp), iters, warmup, stream)
    Cp, Sp = oracle.gemm_points(Xa, Xb, ii, jj, "k", "mn")
    _, w = check(C.float().cpu().double().numpy()[ii, jj], Cp, Sp, "bf16", "NN")
    res.append({"row": "operand layouts", "workload": "4096^3 bf16 NN (B stored [K, N])",
                "kernel_avg_us": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 1),
                "frac": round(flops / t / 1e12 / PEAK_TFLOPS, 4), "bound": "mfma",
                "parity_worst_err_over_bound": round(w, 4)})
    del Ad, Bd

    # fused epilogue: bias along N + GELU
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=0)
    Ad, Bd = A.to(dev), B.to(dev)
    bias = (torch.rand(N, generator=torch.Generator().manual_seed(3)) * 2 - 1).float()
    bd = bias.to(dev)
    epi = _lib.epilogue(1.0, 0.0, bd.data_ptr(), "n", "gelu")
    t = _event_time(lambda: h.run_raw_ex(Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), M, N, K, K,
                                         K, N, 0, 0, epi, sp), iters, warmup, stream)
    Cp, Sp = oracle.gemm_nt_points(A, B, ii, jj)
    Dp = oepi.apply(Cp[None, :], bias=bias.numpy()[jj], bias_along="n", act="gelu")[0]
    _, w = check_epilogue(C.float().cpu().double().numpy()[ii, jj], Dp, Sp,
                          np.abs(bias.numpy()[jj].astype(np.float64)), "bf16", "epilogue")
    res.append({"row": "fused epilogue", "workload": "4096^3 bf16, + bias[n], GELU",
                "kernel_avg_us": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 1),
                "frac": round(flops / t / 1e12 / PEAK_TFLOPS, 4), "bound": "mfma",
                "parity_worst_err_over_bound": round(w, 4)})
    del Ad, Bd, C

    # FP8 E4M3 with per-tensor and with blockwise (1 x 128 / 128 x 128) scales
    for mode in ("tensor", "block"):
        A8, B8, sa, sb = make_fp8_operands(M, N, K, "e4m3", "e4m3", "uniform", seed=0, mode=mode,
                                           block_m=1)
        Ad, Bd, sad, sbd = A8.to(dev), B8.to(dev), sa.to(dev), sb.to(dev)
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        sc = _lib.fp8_scales(mode, sad.data_ptr(), sbd.data_ptr(), 1)
        t = _event_time(lambda: h.run_raw_fp8(3, 3, Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), M,
                                              N, K, K, K, N, 0, sc, None, sp), iters, warmup,
                        stream)
        Cp, Sp = ofp8.gemm_points(A8, B8, ii, jj, K=K, mode=mode, scale_a=sa, scale_b=sb)
        _, w = check(C.float().cpu().double().numpy()[ii, jj], Cp, Sp, "bf16", "fp8")
        res.append({"row": "FP8", "workload": "4096^3 e4m3 x e4m3, %s scales -> bf16" % (
                        "per-tensor" if mode == "tensor" else "1x128 / 128x128 block"),
                    "kernel_avg_us": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 1),
                    "frac": round(flops / t / 1e12 / 5000.0, 4), "bound": "mfma (fp8 5.0 PF)",
                    "parity_worst_err_over_bound": round(w, 4)})
        del Ad, Bd, C

    # grouped: 64 experts with uneven token counts, one launch
    tokens = [64, 17, 200, 3, 90, 128, 256, 40] * 8
    Ng, Kg = 2048, 7168
    ops = [make_operands(m, Ng, Kg, "bf16", "llm", seed=100 + i) for i, m in enumerate(tokens)]
    dops = [(A.to(dev), B.to(dev), torch.empty((A.shape[0], Ng), dtype=torch.bfloat16, device=dev))
            for A, B in ops]
    probs = [_lib.GemmGroupProblem(a.data_ptr(), b.data_ptr(), c.data_ptr(), None, a.shape[0], Ng,
                                   Kg, Kg, Kg, Ng) for a, b, c in dops]
    t = _event_time(lambda: _lib.gemm_run_grouped(h._h, probs, 0, 0, None, sp), iters, warmup,
                    stream)
    gflops = sum(2.0 * m * Ng * Kg for m in tokens)
    worst = 0.0
    for gi in (0, 2, 6, 11):
        A, B = ops[gi]
        mi = rng.integers(0, A.shape[0], 200)
        nj = rng.integers(0, Ng, 200)
        Cp, Sp = oracle.gemm_nt_points(A, B, mi, nj)
        _, w = check(dops[gi][2].float().cpu().double().numpy()[mi, nj], Cp, Sp, "bf16", "grouped")
        worst = max(worst, w)
    # each expert's weights are read once, so at ~100 tokens per expert the
    # launch sits below the ridge point: priced against HBM
    gbytes = sum(2.0 * (m * Kg + Ng * Kg + m * Ng) for m in tokens)
    hbm_bound = gflops / gbytes < PEAK_TFLOPS / HBM_TBS
    res.append({"row": "grouped GEMM", "workload": "64 experts, %d tokens, N=%d K=%d bf16, one launch"
                % (sum(tokens), Ng, Kg),
                "kernel_avg_us": round(t * 1e6, 2), "tflops": round(gflops / t / 1e12, 1),
                "gbs": round(gbytes / t / 1e9, 1),
                "frac": round(gbytes / t / 1e12 / HBM_TBS if hbm_bound else gflops / t / 1e12 / PEAK_TFLOPS, 4),
                "bound": "hbm" if hbm_bound else "mfma",
                "parity_worst_err_over_bound": round(worst, 4)})
    h.close()
    return res


# Every configured workload: (name, M, N, K, in, out, values, rotating input
# sets).  The sets rotate so that the operands of one launch are not in the
# 256 MB last-level cache from the launch before (sets x algorithmic bytes
# >= 512 MB, or one set when a single one is larger).
CONFIGS = [
    ("square512", 512, 512, 512, "bf16", "fp32", "uniform", 8),
    ("square4096", 4096, 4096, 4096, "bf16", "bf16", "uniform", 6),
    ("square4096_fp16", 4096, 4096, 4096, "fp16", "bf16", "uniform", 6),
    ("prefill8192", 8192, 8192, 8192, "bf16", "bf16", "llm", 2),
    ("prefill_mlp_up", 8192, 28672, 8192, "bf16", "bf16", "llm", 1),
    ("decode_mlp_up", 256, 28672, 8192, "bf16", "bf16", "llm", 2),
    ("decode_mlp_down", 256, 8192, 28672, "bf16", "bf16", "llm", 2),
    ("decode_qkv", 256, 10240, 8192, "bf16", "bf16", "llm", 3),
    ("decode_attn_out", 256, 8192, 8192, "bf16", "bf16", "llm", 4),
    ("ragged_1000x4097x1536", 1000, 4097, 1536, "fp16", "fp32", "uniform", 16),
    ("ragged_127x28672x8192", 127, 28672, 8192, "fp16", "fp32", "uniform", 2),
    ("ragged_3000x3000x5000", 3000, 3000, 5000, "fp16", "fp32", "uniform", 6),
    ("ragged_1x8192x8192", 1, 8192, 8192, "fp16", "fp32", "uniform", 4),
]


def _pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    pos = (len(xs) - 1) * q
    lo = int(pos)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (pos - lo)


def time_config(g, cfg, iters=50, warmup=10, check=True):
    """One configured workload: `iters` launches, each between two HIP events on
    the launch stream, after a 0.3 s settle phase and `warmup` launches.  Returns
    median / p10 / p90 of the per-launch times, the batch mean (first to last
    event), TFLOP/s and roofline fraction at the median, the plan, and an oracle
    spot check (two whole rows and 2000 points of the last output)."""
    import torch
    from gemm_inputs import make_operands
    from dense_gemm_nt_amd import roofline
    name, M, N, K, in_dt, out_dt, dist, sets = cfg
    dev = torch.device("cuda", 0)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    code = {"bf16": 0, "fp16": 1, "fp32": 2}
    bufs = []
    for i in range(sets):
        A, B = make_operands(M, N, K, in_dt, dist, seed=i)
        bufs.append((A.to(dev), B.to(dev), torch.empty((M, N), dtype=tdt[out_dt], device=dev)))
        del A, B
    h = g.Gemm()
    stream = torch.cuda.Stream(device=dev)
    sp = stream.cuda_stream
    n_launch = [0]

    def launch():
        A, B, C = bufs[n_launch[0] % sets]
        h.run_raw(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, K, K, N,
                  code[in_dt], code[out_dt], sp)
        n_launch[0] += 1

    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            for _ in range(10):
                launch()
            torch.cuda.synchronize()
        for _ in range(warmup):
            launch()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for e0, e1 in ev:
            e0.record(stream)
            launch()
            e1.record(stream)
        torch.cuda.synchronize()
    us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
    batch_us = ev[0][0].elapsed_time(ev[-1][1]) * 1e3 / iters
    last = (n_launch[0] - 1) % sets
    plan = g.gemm_plan(M, N, K, code[in_dt], code[out_dt])
    r = roofline.roofline(M, N, K, 2, 4 if out_dt == "fp32" else 2, peak_tflops=PEAK_TFLOPS,
                          hbm_tbs=HBM_TBS)
    med = _pct(us, 0.5)
    flops = 2.0 * M * N * K
    floor_us = max(flops / (PEAK_TFLOPS * 1e12), r.bytes / (HBM_TBS * 1e12)) * 1e6
    rec = {"config": name, "M": M, "N": N, "K": K, "in": in_dt, "out": out_dt, "values": dist,
           "sets": sets, "iters": iters,
           "median_us": round(med, 2), "p10_us": round(_pct(us, 0.1), 2),
           "p90_us": round(_pct(us, 0.9), 2), "batch_mean_us": round(batch_us, 2),
           "tflops": round(flops / (med * 1e-6) / 1e12, 1),
           "pct_mfma_peak": round(100 * flops / (med * 1e-6) / 1e12 / PEAK_TFLOPS, 2),
           "bound": r.bound, "floor_us": round(floor_us, 2),
           "roofline_frac": round(floor_us / med, 4),
           "plan": {"name": plan["name"], "splits": plan["splits"], "streamk": plan["streamk"],
                    "workgroups": plan["workgroups"]}}
    if r.bound == "hbm":
        rec["gbs"] = round(r.bytes / (med * 1e-6) / 1e9, 1)
    rec["traffic"] = traffic_for("%dx%dx%d %s->%s" % (M, N, K, in_dt, out_dt), plan)
    if check:
        t0 = time.perf_counter()
        rec["parity_worst_err_over_bound"] = round(
            spot_check([(None, None, bufs[last][2])], 0, (M, N, K), in_dt, out_dt, dist,
                       seed=last), 4)
        rec["oracle_check_s"] = round(time.perf_counter() - t0, 2)
    h.close()
    del bufs
    torch.cuda.empty_cache()
    return rec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shapes, in_dt, dist, target_s=10.0):
    """The oracle as it is, on whole rows of the same workload, on this host's
    cores: about `target_s` seconds of work (more rows, or repeats of the whole
    product once every row fits in less)."""
    import oracle
    from gemm_inputs import make_operands
    M, N, K = shapes
    A, B = make_operands(M, N, K, in_dt, dist, seed=0)
    rows = 16
    while True:
        t0 = time.perf_counter()
        oracle.gemm_nt_rows(A, B, list(range(rows)), K=K, in_dtype=in_dt)
        dt = time.perf_counter() - t0
        if dt >= target_s or rows >= M:
            break
        rows = min(M, max(rows * 2, int(rows * target_s / max(dt, 1e-3) * 1.1)))
    reps = 1
    if dt < target_s:
        # every row took less than the target: repeat the whole product
        reps = max(1, int(target_s / max(dt, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.gemm_nt_rows(A, B, list(range(rows)), K=K, in_dtype=in_dt)
        dt = (time.perf_counter() - t0) / reps
    flops = 2.0 * rows * N * K
    if rows < M:
        sample = "%d of %d output rows of the %dx%dx%d product (%.1f GFLOP) in %.1f s" % (
            rows, M, M, N, K, flops / 1e9, dt)
    else:
        sample = "the whole %dx%dx%d product (%.1f GFLOP), %d time%s in %.1f s" % (
            M, N, K, flops / 1e9, reps, "s" if reps > 1 else "", dt * reps)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": sample, "cpu_model": cpu_model(),
            "per_core": per_core_rate()}


def per_core_rate():
    """The oracle on one thread (a child process with OMP_NUM_THREADS=1): the
    whole 512^3 BF16 product, GFLOP/s per core."""
    import subprocess
    code = ("import time, sys; sys.path.insert(0, %r); import oracle; "
            "from gemm_inputs import make_operands; "
            "A, B = make_operands(512, 512, 512, 'bf16', 'uniform', seed=0); "
            "oracle.gemm_nt(A[:8], B); t = time.perf_counter(); oracle.gemm_nt(A, B); "
            "print(2 * 512 ** 3 / (time.perf_counter() - t) / 1e9, oracle.num_threads())" % ROOT)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                             text=True, timeout=120, check=True).stdout.split()
        return {"gflops": round(float(out[0]), 3), "threads": int(out[1]),
                "sample": "the whole 512^3 bf16 product"}
    except (subprocess.SubprocessError, ValueError, IndexError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-check", action="store_true", help="skip the parity spot check")
    ap.add_argument("--quick", action="store_true", help="primary workload only")
    ap.add_argument("--all-configs", action="store_true",
                    help="one JSON line per configured workload (median / p10 / p90 of 50 "
                         "event-timed launches each), then exit")
    ap.add_argument("--config", action="append", default=[],
                    help="with --all-configs: only the named workload(s)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GEMM has no multi-GPU path here "
              "(rerun with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_gemm_nt_amd as g
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    from dense_gemm_nt_amd import roofline

    if args.all_configs:
        for cfg in CONFIGS:
            if args.config and cfg[0] not in args.config:
                continue
            print(json.dumps(time_config(g, cfg, check=not args.no_check)), flush=True)
        return

    # primary: 4096^3 bf16 -> bf16, six rotating input sets (6 x 96 MB > 256 MB cache)
    shapes = (4096, 4096, 4096)
    wall_ms, event_ms, bufs, last, settle = time_gemm(g, shapes, args.steps, args.warmup, 6,
                                                      "bf16", "bf16", "uniform")
    worst = None if args.no_check else spot_check(bufs, last, shapes, "bf16", "bf16", "uniform")
    del bufs
    torch.cuda.empty_cache()
    M, N, K = shapes
    flops = 2.0 * M * N * K
    plan = g.gemm_plan(M, N, K, 0, 0)
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (event_ms * 1e-3) / 1e12
    out = {
        "metric": "TFLOP/s & % MFMA peak, BF16 GEMM at 4096^3 and 256x28672x8192",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: A, B uniform[-1,1) rounded to bf16, seeds 0..5 rotating",
        "config": {"workload": "gemm_nt M=N=K=4096 bf16 in, fp32 accumulate, bf16 out",
                   "M": M, "N": N, "K": K, "plan": plan["name"],
                   "pct_mfma_peak": round(100 * value / PEAK_TFLOPS, 2),
                   "cache": "cold: 6 rotating input sets (576 MB)",
                   "settle_launches": settle,
                   "parity_worst_err_over_bound": worst},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": traffic_for("4096x4096x4096 bf16->bf16", plan),
                     "kernel_avg_us": round(event_ms * 1e3, 3)},
    }

    if not args.quick:
        # decode-regime shape from the same metric: HBM-bound on this machine
        d = (256, 28672, 8192)
        w2, e2, bufs, last, _ = time_gemm(g, d, max(20, args.steps // 2), args.warmup, 2,
                                          "bf16", "bf16", "llm")
        worst2 = None if args.no_check else spot_check(bufs, last, d, "bf16", "bf16", "llm")
        del bufs
        torch.cuda.empty_cache()
        r = roofline.roofline(*d, 2, 2, peak_tflops=PEAK_TFLOPS, hbm_tbs=HBM_TBS)
        tf = 2.0 * d[0] * d[1] * d[2] / (e2 * 1e-3) / 1e12
        gbs = r.bytes / (e2 * 1e-3) / 1e9
        out["secondary"] = {
            "workload": "gemm_nt M=256 N=28672 K=8192 bf16->bf16 (decode MLP-up)",
            "plan": g.gemm_plan(*d, 0, 0)["name"],
            "splits": g.gemm_plan(*d, 0, 0)["splits"],
            "ms_per_step": round(w2, 5),
            "tflops": round(2.0 * d[0] * d[1] * d[2] / (w2 * 1e-3) / 1e12, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_TBS * 1000,
                         "unit": "GB/s", "frac": round(gbs / (HBM_TBS * 1000), 4),
                         "kernel_avg_us": round(e2 * 1e3, 3), "kernel_tflops": round(tf, 2),
                         "traffic": traffic_for("256x28672x8192 bf16->bf16",
                                                g.gemm_plan(*d, 0, 0))},
            "parity_worst_err_over_bound": worst2,
        }

    if not args.quick:
        out["extensions"] = extensions(g)
        torch.cuda.empty_cache()
        # every configured workload, 50 event-timed launches each
        out["configs"] = [time_config(g, cfg, check=not args.no_check) for cfg in CONFIGS]

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(shapes, "bf16", "uniform")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
