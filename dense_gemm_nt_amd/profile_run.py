"""Workload driver for rocprofv3 runs (kernel traces and hardware counters).

    rocprofv3 --kernel-trace --stats -d OUT -o run -- python -m dense_gemm_nt_amd.profile_run --workload square4096
    rocprofv3 --pmc FETCH_SIZE -d OUT -o fetch -- python -m dense_gemm_nt_amd.profile_run --workload square4096

Runs `--iters` GEMM launches on rotating synthetic input sets, then one plain
device-to-device copy of `--copy-mb` MiB: a kernel of known traffic (reads and
writes copy-mb MiB each) that calibrates the byte counters.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WORKLOADS = {
    # name: (M, N, K, in, out, dist, rotating sets)
    "square512": (512, 512, 512, "bf16", "fp32", "uniform", 8),
    "square4096": (4096, 4096, 4096, "bf16", "bf16", "uniform", 6),
    "square4096_fp16": (4096, 4096, 4096, "fp16", "bf16", "uniform", 6),
    "prefill8192": (8192, 8192, 8192, "bf16", "bf16", "llm", 2),
    "prefill_mlp_up": (8192, 28672, 8192, "bf16", "bf16", "llm", 1),
    "decode_mlp_up": (256, 28672, 8192, "bf16", "bf16", "llm", 2),
    "decode_mlp_down": (256, 8192, 28672, "bf16", "bf16", "llm", 2),
    "decode_qkv": (256, 10240, 8192, "bf16", "bf16", "llm", 3),
    "decode_attn_out": (256, 8192, 8192, "bf16", "bf16", "llm", 4),
    "ragged_1000x4097x1536": (1000, 4097, 1536, "fp16", "fp32", "uniform", 8),
    "ragged_127x28672x8192": (127, 28672, 8192, "fp16", "fp32", "uniform", 2),
    "ragged_3000x3000x5000": (3000, 3000, 5000, "fp16", "fp32", "uniform", 6),
    "ragged_1x8192x8192": (1, 8192, 8192, "fp16", "fp32", "uniform", 4),
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="square4096", choices=sorted(WORKLOADS))
    ap.add_argument("--iters", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--copy-mb", type=int, default=512)
    args = ap.parse_args()

    import torch
    import dense_gemm_nt_amd as g
    from gemm_inputs import make_operands

    M, N, K, ind, outd, dist, sets = WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    code = {"bf16": 0, "fp16": 1, "fp32": 2}
    bufs = []
    for i in range(sets):
        A, B = make_operands(M, N, K, ind, dist, seed=i)
        bufs.append((A.to(dev), B.to(dev), torch.empty((M, N), dtype=tdt[outd], device=dev)))
    h = g.Gemm()
    s = torch.cuda.current_stream(dev).cuda_stream
    for i in range(args.warmup + args.iters):
        A, B, C = bufs[i % sets]
        h.run_raw(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, K, K, N, code[ind], code[outd], s)
    torch.cuda.synchronize()
    n = args.copy_mb << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print("profile_run %s: %d launches of %s, copy %d MiB" % (args.workload, args.warmup + args.iters,
                                                            g.gemm_plan(M, N, K, code[ind], code[outd])["name"],
                                                            args.copy_mb), flush=True)


if __name__ == "__main__":
    main()
