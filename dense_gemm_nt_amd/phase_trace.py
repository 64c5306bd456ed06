"""Phase trace of the 256x256 ping-pong kernel: where a slab's cycles go.

    python -m dense_gemm_nt_amd.phase_trace --build       # CPU: the instrumented library
    python -m dense_gemm_nt_amd.phase_trace [--shape 4096,4096,4096] [--dtype bf16]
                                            [--out FILE.md]   # GPU

The instrumented copy (libgemm_nt_trace.so, built with -DGNT_PP2_TRACE; the
hooks are described in csrc/gemm_nt_trace.hpp) records the shader clock at five
points of every slab iteration of each wave, for slabs 16..31 of blocks 0..31.
This driver runs one 16-bit shape through both libraries on rotating input
sets, checks that the traced copy gives the library's bits, times both (the
trace's own cost), and prints per-quantity medians in shader-clock cycles:
each group's memory phase (direct-to-LDS loads and fragment reads), compute
phase (issue of its 32 MFMAs), the wait for its loads, the two barrier waits,
and the slab period against the 2048-cycle MFMA ideal (64 MFMAs of 32 cycles
per SIMD and slab).  Only the plain 16-bit kernels are traced (the
instrumented blockwise-FP8 and persistent kernels spill).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PKG = os.path.dirname(os.path.abspath(__file__))
TRACE_LIB = os.path.join(PKG, "libgemm_nt_trace.so")
T0, TN, REC, BLOCKS = 16, 16, 6, 32          # as in csrc/gemm_nt_trace.hpp
TRACE_BYTES = BLOCKS * 8 * TN * REC * 8
CODE = {"bf16": 0, "fp16": 1}
ROWS = (("period", "slab period (e0 to the next e0)"),
        ("g0_mem", "group 0 memory phase: B loads + 24 fragment reads (e0-e1)"),
        ("g0_bar1", "group 0 waits at the barrier ending it (e1-e2)"),
        ("g0_comp", "group 0 compute phase: MFMA issue (e2-e3)"),
        ("g0_vmw", "group 0 waits for its B loads (e3-e4)"),
        ("g0_bar2", "group 0 waits at the barrier ending it (e4-next e0)"),
        ("g1_comp", "group 1 compute phase: MFMA issue (e0-e1)"),
        ("g1_bar1", "group 1 waits at the barrier ending it (e1-e2)"),
        ("g1_mem", "group 1 memory phase: A loads + 24 fragment reads (e2-e3)"),
        ("g1_vmw", "group 1 waits for its A loads (e3-e4)"),
        ("g1_bar2", "group 1 waits at the barrier ending it (e4-next e0)"))


def build():
    from dense_gemm_nt_amd import build as b
    return b.build(out=TRACE_LIB, defines=["-DGNT_PP2_TRACE"])


def _lib(path):
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L = ctypes.CDLL(path)
    L.gemm_create.argtypes = [ctypes.POINTER(vp)]
    L.gemm_run.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, ci, vp]
    L.gemm_destroy.argtypes = [vp]
    h = vp()
    if L.gemm_create(ctypes.byref(h)) != 0:
        raise RuntimeError("gemm_create failed for %s" % path)
    return L, h


def _pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(q * len(v)))]


def analyse(tr):
    """tr[block][wave][slab] = [e0..e4, reference clock at e0] -> per-quantity
    lists of cycle counts, and the shader clock in GHz."""
    rows = {k: [] for k, _ in ROWS}
    ghz = []
    for blk in tr:
        for w, ev in enumerate(blk):
            if ev[0][0] == 0:
                continue
            if ev[-1][5] > ev[0][5]:
                ghz.append((ev[-1][0] - ev[0][0]) / ((ev[-1][5] - ev[0][5]) / 100e6) / 1e9)
            for i in range(len(ev) - 1):
                e, n = ev[i], ev[i + 1]
                rows["period"].append(n[0] - e[0])
                if w < 4:
                    rows["g0_mem"].append(e[1] - e[0])
                    rows["g0_bar1"].append(e[2] - e[1])
                    rows["g0_comp"].append(e[3] - e[2])
                    rows["g0_vmw"].append(e[4] - e[3])
                    rows["g0_bar2"].append(n[0] - e[4])
                else:
                    rows["g1_comp"].append(e[1] - e[0])
                    rows["g1_bar1"].append(e[2] - e[1])
                    rows["g1_mem"].append(e[3] - e[2])
                    rows["g1_vmw"].append(e[4] - e[3])
                    rows["g1_bar2"].append(n[0] - e[4])
    return rows, (_pct(ghz, 0.5) if ghz else float("nan"))


def run(M, N, K, dtype, rounds=3, iters=40):
    import torch
    import dense_gemm_nt_amd as g
    from gemm_inputs import make_operands
    if not os.path.exists(TRACE_LIB):
        raise SystemExit("build the instrumented library first: python -m dense_gemm_nt_amd.phase_trace --build")
    plan = g.gemm_plan(M, N, K, CODE[dtype], 0)
    if plan["name"] != "256x256x64_w8_pp2":
        raise SystemExit("%dx%dx%d runs on %s, not the ping-pong tile" % (M, N, K, plan["name"]))
    dev = torch.device("cuda", 0)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    sets = []
    for s in range(4):
        A, B = make_operands(M, N, K, dtype, "uniform", seed=s)
        sets.append((A.to(dev), B.to(dev)))
    extra = TRACE_BYTES // 2
    C = torch.zeros(M * N + extra, dtype=torch.bfloat16, device=dev)      # C and the trace area
    C0 = torch.empty(M * N, dtype=torch.bfloat16, device=dev)
    Lt, ht = _lib(TRACE_LIB)
    L0, h0 = _lib(os.path.join(PKG, "libgemm_nt.so"))
    stream = torch.cuda.Stream(device=dev)

    def launch(L, h, out, k):
        A, B = sets[k % 4]
        st = L.gemm_run(h, A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, K, K, N,
                        CODE[dtype], 0, ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError("gemm_run returned %d" % st)

    def timed(L, h, out):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        with torch.cuda.stream(stream):
            for k, (e0, e1) in enumerate(ev):
                e0.record(stream)
                launch(L, h, out, k)
                e1.record(stream)
        torch.cuda.synchronize()
        return _pct([a.elapsed_time(b) * 1e3 for a, b in ev], 0.5)

    print("case phase trace %dx%dx%d %s" % (M, N, K, dtype), flush=True)
    times = []
    for _ in range(rounds):
        times.append((timed(Lt, ht, C), timed(L0, h0, C0)))
    with torch.cuda.stream(stream):
        launch(Lt, ht, C, 0)
        launch(L0, h0, C0, 0)
    torch.cuda.synchronize()
    same = bool(torch.equal(C[:M * N].view(torch.int16), C0.view(torch.int16)))
    tr = C[M * N:].view(torch.int64).cpu().view(BLOCKS, 8, TN, REC).tolist()
    Lt.gemm_destroy(ht)
    L0.gemm_destroy(h0)
    return plan, times, same, tr


def report(M, N, K, dtype, plan, times, same, tr):
    rows, ghz = analyse(tr)
    t_tr = _pct([a for a, _ in times], 0.5)
    t_lib = _pct([b for _, b in times], 0.5)
    md = ["# Phase trace of the ping-pong kernel: %dx%dx%d %s -> bf16" % (M, N, K, dtype), "",
          "Command (from the repository root; the instrumented library is built on the CPU first):", "",
          "    python -m dense_gemm_nt_amd.phase_trace --build",
          "    python -m dense_gemm_nt_amd.phase_trace --shape %d,%d,%d --dtype %s" % (M, N, K, dtype), "",
          "Plan %s, %d split%s.  Traced copy %.2f us against the library's %.2f us (median of %d "
          "event-timed launches per round, %d rounds: the trace's own cost); same bits as the "
          "library: %s.  Shader clock %.2f GHz (clock reads over the 100 MHz reference)." % (
              plan["name"], plan["splits"], "s" if plan["splits"] > 1 else "", t_tr, t_lib, 40,
              len(times), "yes" if same else "NO", ghz), "",
          "Cycles (shader clock) over slabs %d..%d of blocks 0..%d, every wave:" % (T0, T0 + TN - 1, BLOCKS - 1), "",
          "| quantity | median | p10 | p90 |", "|---|---|---|---|"]
    for k, label in ROWS:
        v = rows[k]
        md.append("| %s | %d | %d | %d |" % (label, _pct(v, 0.5), _pct(v, 0.1), _pct(v, 0.9)))
    per = _pct(rows["period"], 0.5)
    md += ["", "The MFMA ideal is 2048 cycles per slab; the median period is %.2f times that." % (per / 2048.0), ""]
    return "\n".join(md)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--build", action="store_true")
    ap.add_argument("--shape", default="4096,4096,4096")
    ap.add_argument("--dtype", default="bf16", choices=sorted(CODE))
    ap.add_argument("--out")
    args = ap.parse_args()
    if args.build:
        print(build())
        return
    M, N, K = (int(x) for x in args.shape.split(","))
    text = report(M, N, K, args.dtype, *run(M, N, K, args.dtype))
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)


if __name__ == "__main__":
    main()
