"""Timings behind the planner's rules: each named sweep runs the shapes a rule
decides between, under every alternative the rule weighs, interleaved in one
process (one library handle per alternative; rounds of event-timed launches
taken in turn, each round starting with another alternative, so that a clock
or temperature drift and the order within a round favour none of them).

    python -m dense_gemm_nt_amd.plan_sweep [--sweeps a,b] [--rounds 8] [--out FILE.md]

An alternative is a forced configuration, a forced K split count, or one of the
handle's switches (GEMM_STREAMK, GEMM_INREDUCE, GEMM_ROTATE), set while its handle is
created.  Inputs rotate over enough sets to read cold, as in bench.py.  Prints one JSON line per (shape, alternative) with the median, p10
and p90 over all rounds, marks the planner's own choice, and writes a Markdown
table per sweep to --out.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PP2, W4_256x128 = "256x256x64_w8_pp2", "256x128x64_w4_u8"
T128, T128_S2, T32 = "128x128x64_w8_s4", "128x128x64_w8_s2", "32x128x64_w4_s6"

# name: (what the rule decides, shapes (M, N, K, in, out, value distribution),
#        alternatives (label, environment))
SWEEPS = {
    "decode_tile": (
        "M = 256: the 256x256 ping-pong tile, or the four-wave 256x128 tile when the "
        "ping-pong tile would need more than four K splits with K <= 16384",
        [(256, 10240, 8192, "bf16", "bf16", "llm"), (256, 8192, 8192, "bf16", "bf16", "llm"),
         (256, 28672, 8192, "bf16", "bf16", "llm"), (256, 8192, 28672, "bf16", "bf16", "llm")],
        [("plan", {}), (PP2, {"GEMM_CONFIG": PP2}), (W4_256x128, {"GEMM_CONFIG": W4_256x128})]),
    "decode_fill": (
        "128 < M <= 256: a 256-row tile only while its blocks fill the machine as well as the "
        "128x128 tile's would; the four-wave tile over the ping-pong tile when it fills more",
        [(192, 4096, 4096, "bf16", "bf16", "llm"), (256, 4096, 4096, "bf16", "bf16", "llm"),
         (256, 8192, 2048, "bf16", "bf16", "llm"), (256, 2048, 8192, "bf16", "bf16", "llm"),
         (200, 6144, 3072, "bf16", "bf16", "llm"), (256, 8192, 4096, "bf16", "bf16", "llm"),
         (256, 16384, 4096, "bf16", "bf16", "llm"), (256, 28672, 4096, "bf16", "bf16", "llm"),
         (160, 4096, 8192, "bf16", "bf16", "llm")],
        [("plan", {}), (T128, {"GEMM_CONFIG": T128}), (W4_256x128, {"GEMM_CONFIG": W4_256x128}),
         (PP2, {"GEMM_CONFIG": PP2})]),
    "mid_fill": (
        "M > 256: the 128x128 tile, where its tiles fit one pass, when it fills that pass at "
        "least as well as the ping-pong tile fills its own",
        [(768, 4096, 4096, "bf16", "bf16", "llm"), (384, 8192, 4096, "bf16", "bf16", "llm"),
         (640, 2048, 8192, "bf16", "bf16", "llm"), (512, 16384, 2048, "bf16", "bf16", "llm"),
         (512, 8192, 8192, "bf16", "bf16", "llm"), (768, 8192, 2048, "bf16", "bf16", "llm")],
        [("plan", {}), (T128, {"GEMM_CONFIG": T128}), (PP2, {"GEMM_CONFIG": PP2})]),
    "small_tile_fill": (
        "M > 64: the 32x128 tile where the 128x128 tile was chosen but the 32-row tiles, in one "
        "pass with their own K splits, fill the machine strictly better",
        [(178, 640, 2240, "bf16", "bf16", "llm"), (74, 1408, 512, "bf16", "bf16", "llm"),
         (618, 704, 3968, "bf16", "bf16", "llm"), (640, 768, 8192, "bf16", "bf16", "llm"),
         (192, 4096, 4096, "bf16", "bf16", "llm"), (96, 8192, 8192, "bf16", "bf16", "llm")],
        [("plan", {}), (T32, {"GEMM_CONFIG": T32}), (T128, {"GEMM_CONFIG": T128})]),
    "small_m": (
        "M <= 64: the 32x128 tile while its tiles fit one pass of the machine (M <= 32 always); "
        "from M = 96, or past one pass, the 128x128 tile",
        [(m, 8192, 8192, "bf16", "bf16", "llm") for m in (1, 16, 32, 64, 96, 128)] +
        [(40, 28672, 8192, "bf16", "bf16", "llm"), (64, 28672, 8192, "bf16", "bf16", "llm"),
         (32, 28672, 8192, "bf16", "bf16", "llm"), (64, 4096, 4096, "bf16", "bf16", "llm")],
        [("plan", {}), (T32, {"GEMM_CONFIG": T32}), (T128, {"GEMM_CONFIG": T128})]),
    "small_square": (
        "small squares: the 32x128 tile when, in one pass with its K splits, it fills the "
        "machine strictly better than the 128x128 tile with its splits",
        [(n, n, n, "bf16", "fp32", "uniform") for n in (512, 768, 1024, 1536, 2048)],
        [("plan", {}), (T32, {"GEMM_CONFIG": T32}), (T128, {"GEMM_CONFIG": T128}),
         (PP2, {"GEMM_CONFIG": PP2})]),
    "two_blocks_per_cu": (
        "128x128 tiles that overflow one pass of the machine but fit two: the "
        "two-stage ring, two blocks per compute unit",
        [(1000, 4097, 1536, "fp16", "fp32", "uniform"), (1024, 4096, 2048, "bf16", "bf16", "uniform"),
         (1500, 2900, 1024, "bf16", "bf16", "uniform")],
        [("plan", {}), (T128, {"GEMM_CONFIG": T128}), (T128_S2, {"GEMM_CONFIG": T128_S2}),
         (PP2, {"GEMM_CONFIG": PP2})]),
    "small_m_fill": (
        "M <= 32: K splits for about three quarters of the compute units (rounded), "
        "not all of them",
        [(1, 4096, 16384, "bf16", "bf16", "llm"), (1, 2048, 32768, "bf16", "bf16", "llm"),
         (16, 4096, 4096, "bf16", "bf16", "llm"), (1, 4096, 8192, "bf16", "bf16", "llm")],
        [("plan", {})] + [("%s splits=%d" % (T32, s), {"GEMM_CONFIG": T32, "GEMM_SPLITS": str(s)})
                          for s in (4, 5, 8, 16)]),
    "split_stride": (
        "M <= 32 with K splits: split counts whose starts are a multiple of 4 KB "
        "apart are moved to the nearest count that is not",
        [(1, 8192, 8192, "fp16", "fp32", "uniform"), (32, 8192, 8192, "bf16", "bf16", "llm"),
         (1, 4096, 16384, "bf16", "bf16", "llm")],
        [("plan", {})] + [("%s splits=%d" % (T32, s), {"GEMM_CONFIG": T32, "GEMM_SPLITS": str(s)})
                          for s in (2, 3, 4, 5)]),
    "stream_k": (
        "stream-K over all compute units when the ping-pong tiles with their K splits "
        "leave at least 3/8 of them idle and a run holds at least 32 k-slabs",
        [(3000, 3000, 5000, "fp16", "fp32", "uniform"), (2304, 2304, 8192, "bf16", "bf16", "uniform"),
         (3000, 3000, 1536, "fp16", "fp32", "uniform")],
        [("plan", {}), ("stream-K off", {"GEMM_STREAMK": "0"}), ("stream-K on", {"GEMM_STREAMK": "2"})]),
    "decode_splits": (
        "few-tile decode shapes: the four-wave tile's three or four K splits with a second "
        "pass, against two splits reduced in the kernel, and against one split",
        [(256, 10240, 8192, "bf16", "bf16", "llm"), (256, 8192, 8192, "bf16", "bf16", "llm"),
         (256, 8192, 28672, "bf16", "bf16", "llm")],
        [("plan", {}), ("%s 2 splits" % W4_256x128, {"GEMM_CONFIG": W4_256x128, "GEMM_SPLITS": "2"}),
         ("%s 1 split" % W4_256x128, {"GEMM_CONFIG": W4_256x128, "GEMM_SPLITS": "1"}),
         ("%s 2 splits" % PP2, {"GEMM_CONFIG": PP2, "GEMM_SPLITS": "2"})]),
    "mid_four_wave": (
        "mid-size shapes: the planned tile against the four-wave 256x128 tile, whose "
        "wave blocks read fewer LDS bytes per FLOP",
        [(1000, 4097, 1536, "fp16", "fp32", "uniform"), (1024, 4096, 2048, "bf16", "bf16", "uniform"),
         (1500, 2900, 1024, "bf16", "bf16", "uniform"), (1536, 1536, 1536, "bf16", "fp32", "uniform"),
         (2048, 2048, 2048, "bf16", "fp32", "uniform"), (127, 28672, 8192, "fp16", "fp32", "uniform"),
         (3000, 3000, 5000, "fp16", "fp32", "uniform")],
        [("plan", {}), (W4_256x128, {"GEMM_CONFIG": W4_256x128})]),
    "slab_rotation": (
        "the 32x128 and 128x128 tiles: each 256-column block of tiles starting its k-slabs at a "
        "rotated slab when M <= 128, against walking K from the first slab, and against rotation "
        "at every M (the 256-row tiles always walk K in order)",
        [(1, 8192, 8192, "bf16", "bf16", "llm"), (32, 8192, 8192, "bf16", "bf16", "llm"),
         (64, 8192, 8192, "bf16", "bf16", "llm"), (1, 4096, 16384, "bf16", "bf16", "llm"),
         (1, 2048, 32768, "bf16", "bf16", "llm"), (96, 8192, 8192, "bf16", "bf16", "llm"),
         (128, 8192, 8192, "bf16", "bf16", "llm"), (127, 28672, 8192, "fp16", "fp32", "uniform"),
         (1024, 1024, 1024, "bf16", "fp32", "uniform"), (1000, 4097, 1536, "fp16", "fp32", "uniform"),
         (1500, 2900, 1024, "bf16", "bf16", "uniform"), (2048, 2048, 2048, "bf16", "fp32", "uniform")],
        [("plan", {}), ("natural order", {"GEMM_ROTATE": "0"}), ("rotated", {"GEMM_ROTATE": "2"})]),
    "in_kernel_reduction": (
        "K splits reduced in the kernel by the last split of a tile to finish (two on the "
        "256-row tiles, any number on the 32x128 and 128x128 tiles), instead of a second pass",
        [(256, 28672, 8192, "bf16", "bf16", "llm"), (512, 8192, 8192, "bf16", "bf16", "llm"),
         (1, 8192, 8192, "bf16", "bf16", "llm"), (16, 4096, 4096, "bf16", "bf16", "llm"),
         (1, 2048, 32768, "bf16", "bf16", "llm"), (64, 8192, 8192, "bf16", "bf16", "llm"),
         (96, 8192, 8192, "bf16", "bf16", "llm"), (128, 8192, 8192, "bf16", "bf16", "llm")],
        [("plan", {}), ("second pass", {"GEMM_INREDUCE": "0"})]),
}

CODE = {"bf16": 0, "fp16": 1, "fp32": 2}
ENV_KEYS = ("GEMM_CONFIG", "GEMM_SPLITS", "GEMM_STREAMK", "GEMM_INREDUCE", "GEMM_PERSIST",
            "GEMM_ROTATE")


def _pct(xs, q):
    xs = sorted(xs)
    pos = (len(xs) - 1) * q
    lo = int(pos)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (pos - lo)


def _handle(g, env):
    old = {k: os.environ.get(k) for k in ENV_KEYS}
    try:
        for k in ENV_KEYS:
            os.environ.pop(k, None)
        os.environ.update(env)
        return g.Gemm()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def input_sets(M, N, K, ind, outd):
    """Rotating input sets for one shape: enough that together they exceed
    600 MB, more than the 256 MB memory-side cache, so every launch reads its
    operands cold, as bench.py's timings do (2 to 16 sets)."""
    b = {"bf16": 2, "fp16": 2, "fp32": 4}
    per = b[ind] * (M * K + N * K) + b[outd] * M * N
    return max(2, min(16, -(-(600 << 20) // per)))


def run_shape(g, shape, alts, rounds, per=20, sets=None):
    import torch
    from gemm_inputs import make_operands
    M, N, K, ind, outd, dist = shape
    if sets is None:
        sets = input_sets(M, N, K, ind, outd)
    dev = torch.device("cuda", 0)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    bufs = []
    for i in range(sets):
        A, B = make_operands(M, N, K, ind, dist, seed=i)
        bufs.append((A.to(dev), B.to(dev), torch.empty((M, N), dtype=tdt[outd], device=dev)))
    hs = [_handle(g, env) for _, env in alts]
    stream = torch.cuda.Stream(device=dev)
    n = [0]

    def launch(h):
        A, B, C = bufs[n[0] % sets]
        h.run_raw(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, K, K, N, CODE[ind],
                  CODE[outd], stream.cuda_stream)
        n[0] += 1

    times = [[] for _ in alts]
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            for h in hs:
                for _ in range(5):
                    launch(h)
            torch.cuda.synchronize()
        for r in range(rounds):
            # each round starts with another alternative, so that a position in
            # the round (what ran just before) favours none of them
            for vi in [(r + k) % len(hs) for k in range(len(hs))]:
                h = hs[vi]
                for _ in range(5):
                    launch(h)
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(per)]
                for e0, e1 in ev:
                    e0.record(stream)
                    launch(h)
                    e1.record(stream)
                torch.cuda.synchronize()
                times[vi] += [a.elapsed_time(b) * 1e3 for a, b in ev]
    for h in hs:
        h.close()
    del bufs
    torch.cuda.empty_cache()
    return [(_pct(t, 0.5), _pct(t, 0.1), _pct(t, 0.9)) for t in times]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--sweeps", default=",".join(SWEEPS))
    ap.add_argument("--rounds", type=int, default=8)
    ap.add_argument("--out", help="Markdown file for the tables")
    args = ap.parse_args()
    import torch  # noqa: F401
    import dense_gemm_nt_amd as g
    md = ["# Plan-rule sweeps", "",
          "Command: `python -m dense_gemm_nt_amd.plan_sweep --sweeps %s --rounds %d`" % (
              args.sweeps, args.rounds), "",
          "Median / p10 / p90 in us over %d interleaved rounds of 20 event-timed launches "
          "per alternative, on rotating input sets that together exceed 600 MB (cold "
          "operands, as in bench.py).  `plan` is the library's own choice, named in "
          "brackets." % args.rounds, ""]
    for name in args.sweeps.split(","):
        what, shapes, alts = SWEEPS[name]
        md += ["## %s" % name, "", what + ".", "",
               "| shape | " + " | ".join(a for a, _ in alts) + " |",
               "|---|" + "---|" * len(alts)]
        for shape in shapes:
            M, N, K, ind, outd, _ = shape
            plan = g.gemm_plan(M, N, K, CODE[ind], CODE[outd])
            print("case %s %dx%dx%d %s->%s plan %s splits %d" % (name, M, N, K, ind, outd,
                                                                  plan["name"], plan["splits"]),
                  flush=True)
            res = run_shape(g, shape, alts, args.rounds)
            for (label, _), (med, p10, p90) in zip(alts, res):
                print(json.dumps({"sweep": name, "shape": [M, N, K, ind, outd], "alt": label,
                                  "median_us": round(med, 2), "p10_us": round(p10, 2),
                                  "p90_us": round(p90, 2),
                                  "plan": plan["name"] if label == "plan" else None,
                                  "plan_splits": plan["splits"] if label == "plan" else None}),
                      flush=True)
            best = min(r[0] for r in res)
            cells = []
            for (label, _), (med, p10, p90) in zip(alts, res):
                c = "%.1f (%.1f-%.1f)" % (med, p10, p90)
                if med == best:
                    c = "**" + c + "**"
                if label == "plan":
                    c += " [%s, %d split%s%s]" % (plan["name"], plan["splits"],
                                                  "s" if plan["splits"] > 1 else "",
                                                  ", stream-K" if plan["streamk"] else "")
                cells.append(c)
            md.append("| %dx%dx%d %s->%s | %s |" % (M, N, K, ind, outd, " | ".join(cells)))
        md.append("")
        if args.out:
            with open(args.out, "w") as f:
                f.write("\n".join(md) + "\n")


if __name__ == "__main__":
    main()
