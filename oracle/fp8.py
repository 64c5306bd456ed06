"""CPU oracle for the FP8 GEMM with per-tensor or blockwise scales -- test
infrastructure.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU library never does.

What it computes (the plain definition, in binary64):

    C[i, j] = sum_k  a(i, k) * sa(i, k) * b(j, k) * sb(j, k)

- "CUTLASS Deep Dive: From CuTe Layouts to Blackwell tcgen05", section "FP8
  and Blockwise Scaling": FP8 (E4M3) operands; with blockwise scaling there is
  one scale per (block_m, block_k) tile of A and one per (block_n, block_k)
  tile of B, applied while accumulating instead of one scale per tensor.
  Applying a block's scale to that block's partial sum, as the page describes,
  equals scaling every element of the block (the scale factors out of the
  block's sum), so the oracle dequantizes the operands and takes one plain sum.
- Readings where the page is silent: the scales are FP32; block_k = 128 and
  block_n = 128, block_m = 1 (one scale per row and 128-deep block, the
  activation granularity) or 128; per-tensor scaling is one FP32 value per
  operand.  Both OCP 8-bit formats are decoded: E4M3 (bias 7, no infinities,
  S.1111.111 is NaN, largest 448) and E5M2 (bias 15, IEEE-style infinities and
  NaNs).
- The sum over k is numpy's float64 matrix product of the dequantized
  operands (a library primitive as one step); every product of an FP32 scale
  and an FP8 value is exact in binary64.

Parity pins: tests/test_oracle_fp8_pins.py (exhaustive decode against torch's
float8 types, exact rationals on tiny blockwise cases, closed forms with
per-block powers of two, block-index and axis checks).
"""
from __future__ import annotations

import numpy as np

FORMATS = ("e4m3", "e5m2")
SCALE_MODES = ("tensor", "block")
BLOCK_K = 128
BLOCK_N = 128


def _decode_table(fmt: str) -> np.ndarray:
    """binary64 value of each of the 256 codes, from the format's bit fields."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        if fmt == "e4m3":
            e, m = (c >> 3) & 0xF, c & 0x7
            if e == 0xF and m == 0x7:
                v = np.nan
            elif e == 0:
                v = s * (m / 8.0) * 2.0 ** -6
            else:
                v = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
        elif fmt == "e5m2":
            e, m = (c >> 2) & 0x1F, c & 0x3
            if e == 0x1F:
                v = s * np.inf if m == 0 else np.nan
            elif e == 0:
                v = s * (m / 4.0) * 2.0 ** -14
            else:
                v = s * (1.0 + m / 4.0) * 2.0 ** (e - 15)
        else:
            raise ValueError("unknown FP8 format %r" % (fmt,))
        out[c] = v
    return out


_TABLES = {}


def decode(codes, fmt: str) -> np.ndarray:
    """Exact binary64 values of FP8 codes (uint8 array or torch uint8/float8 tensor)."""
    if fmt not in _TABLES:
        _TABLES[fmt] = _decode_table(fmt)
    return _TABLES[fmt][_codes(codes)]


def _codes(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint8:
            raise TypeError("FP8 codes must be uint8")
        return x
    import torch  # only to view a tensor's bytes
    return x.detach().cpu().contiguous().view(torch.uint8).numpy()


def _f32(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return x.astype(np.float32)
    return x.detach().cpu().to(dtype=__import__("torch").float32).numpy()


def dequantize(codes, fmt, scales, mode, K, block_rows):
    """The operand's binary64 values times their scales: codes [rows, >= K];
    mode "tensor": one scale; "block": scales [ceil(rows / block_rows)][ceil(K / 128)]."""
    x = decode(codes, fmt)[:, :K]
    s = _f32(scales).astype(np.float64)
    if mode == "tensor":
        if s.size != 1:
            raise ValueError("per-tensor scaling takes one value")
        return x * float(s.reshape(()))
    if mode != "block":
        raise ValueError("unknown scale mode %r" % (mode,))
    rows = x.shape[0]
    nkb = -(-K // BLOCK_K)
    nrb = -(-rows // block_rows)
    if s.shape != (nrb, nkb):
        raise ValueError("block scales must be %d x %d, got %r" % (nrb, nkb, s.shape))
    ri = np.arange(rows) // block_rows
    ki = np.arange(K) // BLOCK_K
    return x * s[ri[:, None], ki[None, :]]


def gemm(A, B, K=None, fmt_a="e4m3", fmt_b="e4m3", mode="tensor", scale_a=1.0, scale_b=1.0,
         block_m=1):
    """C_ref, S (S = sum_k |a sa b sb|) for A [M, >= K] and B [N, >= K] FP8 codes."""
    Ac, Bc = _codes(A), _codes(B)
    K = Ac.shape[1] if K is None else K
    if mode == "tensor":
        scale_a = np.asarray([scale_a], dtype=np.float32).reshape(1) if np.isscalar(scale_a) \
            else scale_a
        scale_b = np.asarray([scale_b], dtype=np.float32).reshape(1) if np.isscalar(scale_b) \
            else scale_b
    if block_m not in (1, 128):
        raise ValueError("block_m must be 1 or 128")
    a = dequantize(Ac, fmt_a, scale_a, mode, K, block_m)
    b = dequantize(Bc, fmt_b, scale_b, mode, K, BLOCK_N)
    return a @ b.T, np.abs(a) @ np.abs(b).T


def gemm_points(A, B, ii, jj, K=None, fmt_a="e4m3", fmt_b="e4m3", mode="tensor", scale_a=1.0,
                scale_b=1.0, block_m=1, chunk=512):
    """C_ref[p], S[p] at (ii[p], jj[p]) of the product gemm() defines."""
    Ac, Bc = _codes(A), _codes(B)
    K = Ac.shape[1] if K is None else K
    if mode == "tensor":
        scale_a = np.asarray([scale_a], dtype=np.float32) if np.isscalar(scale_a) else scale_a
        scale_b = np.asarray([scale_b], dtype=np.float32) if np.isscalar(scale_b) else scale_b
    a = dequantize(Ac, fmt_a, scale_a, mode, K, block_m)
    b = dequantize(Bc, fmt_b, scale_b, mode, K, BLOCK_N)
    ii = np.asarray(ii, dtype=np.int64)
    jj = np.asarray(jj, dtype=np.int64)
    C = np.empty(ii.size)
    S = np.empty(ii.size)
    for p0 in range(0, ii.size, chunk):
        ai, bj = a[ii[p0:p0 + chunk]], b[jj[p0:p0 + chunk]]
        C[p0:p0 + chunk] = np.einsum("pk,pk->p", ai, bj)
        S[p0:p0 + chunk] = np.einsum("pk,pk->p", np.abs(ai), np.abs(bj))
    return C, S
