"""Roofline arithmetic for the NT GEMM (host-side measurement model).

The model is the one the pages use: the work is 2 M N K floating-point operations;
the least traffic is reading A and B once and writing C once; a launch can go no
faster than max(compute time at peak, traffic time at the memory bandwidth).
  * "A Blackwell GEMM by Hand in CuTe DSL: TMA, mbarriers, TMEM, and tcgen05",
    section 1 (Two regimes): FLOP count, bytes with 2-byte A, B and C, the
    compute/memory floor, CTA counts per 128x256 tile and waves over the SMs.
  * "Matmul on sm_120", section Roofline: bytes with 2-byte A and B and a 4-byte
    C, and the memory-bound ceiling 2MNK / time.
Both pages' printed figures pin this module (tests/golden/).

MI355X figures used by default: 2500 TFLOP/s dense BF16/FP16 MFMA (the published
figure; 256 CUs x 2.4 GHz x 4096 FLOP per CU-clock is the nominal 2516.6) and
8.0 TB/s HBM3E.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

MI355X_PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}
MI355X_HBM_TBS = 8.0
MI355X_CUS = 256
MI355X_CLOCK_GHZ = 2.4
MI355X_NOMINAL_TFLOPS = MI355X_CUS * MI355X_CLOCK_GHZ * 4096 / 1000.0   # 2516.58

DTYPE_BYTES = {"bf16": 2, "fp16": 2, "fp32": 4}


def flops(M, N, K):
    return 2 * M * N * K


def min_bytes(M, N, K, in_bytes=2, out_bytes=2):
    """A and B read once, C written once."""
    return in_bytes * (M * K + N * K) + out_bytes * M * N


def intensity(M, N, K, in_bytes=2, out_bytes=2):
    return flops(M, N, K) / min_bytes(M, N, K, in_bytes, out_bytes)


@dataclass
class Roofline:
    flops: float
    bytes: float
    intensity: float
    compute_us: float
    memory_us: float
    bound: str          # "mfma" (compute) or "hbm" (memory)
    floor_us: float
    bound_tflops: float


def roofline(M, N, K, in_bytes=2, out_bytes=2, peak_tflops=MI355X_PEAK_TFLOPS["bf16"],
             hbm_tbs=MI355X_HBM_TBS) -> Roofline:
    f = flops(M, N, K)
    b = min_bytes(M, N, K, in_bytes, out_bytes)
    t_c = f / (peak_tflops * 1e12) * 1e6
    t_m = b / (hbm_tbs * 1e12) * 1e6
    bound = "mfma" if t_c >= t_m else "hbm"
    floor = max(t_c, t_m)
    return Roofline(f, b, f / b, t_c, t_m, bound, floor, f / floor / 1e6)


def memory_ceiling_tflops(M, N, K, in_bytes, out_bytes, hbm_tbs):
    """FLOP rate if only the minimum traffic limited the launch."""
    return flops(M, N, K) * hbm_tbs * 1e12 / min_bytes(M, N, K, in_bytes, out_bytes) / 1e12


def ridge(peak_tflops=MI355X_PEAK_TFLOPS["bf16"], hbm_tbs=MI355X_HBM_TBS):
    return peak_tflops / hbm_tbs


def tiles(M, N, BM, BN):
    return math.ceil(M / BM) * math.ceil(N / BN)


def waves(n_tiles, n_units):
    return n_tiles / n_units
