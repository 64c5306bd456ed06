"""Seeded synthetic operands for the NT GEMM ``C = A . B^T``.

This module holds no arithmetic of the GEMM itself: it only draws the operand
values.  Both the CPU oracle's tests and the GPU path's tests and benchmark take
their inputs from here, so the two sides always see the same bits.

Recipe (the same for every caller):
  * a CPU ``torch.Generator`` seeded with ``seed``; A is drawn first, then B;
  * ``uniform``: ``rand * 2 - 1`` in float32 (uniform on [-1, 1)), rounded to the
    16-bit format with round-to-nearest-even (so +-1.0 can occur after rounding);
  * ``llm``: A ~ N(0, 1) (activations), B ~ N(0, 0.02^2) (weights, stored as the
    [out, in] matrix of a linear layer), drawn in float32, then rounded;
  * ``int3``: integers uniform in {-3, ..., 3}, exact in both 16-bit formats;
  * ``ones``: every entry 1.
A leading dimension larger than K leaves padding columns; they are filled with
NaN so that a kernel which reads past column K-1 poisons its result.
"""
from __future__ import annotations

import torch

DISTS = ("uniform", "llm", "int3", "ones")


def _dtype(name):
    if isinstance(name, torch.dtype):
        return name
    name = str(name)
    if name in ("bf16", "bfloat16"):
        return torch.bfloat16
    if name in ("fp16", "f16", "float16", "half"):
        return torch.float16
    raise ValueError("unknown input format %r" % name)


def _draw(shape, dist, role, g):
    if dist == "uniform":
        return torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    if dist == "llm":
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        return x if role == "A" else x * 0.02
    if dist == "int3":
        return torch.randint(-3, 4, shape, generator=g, dtype=torch.int64).to(torch.float32)
    if dist == "ones":
        return torch.ones(shape, dtype=torch.float32)
    raise ValueError("unknown distribution %r" % dist)


def make_operands(M, N, K, dtype="bf16", dist="uniform", seed=0, lda=None, ldb=None):
    """Return (A_store, B_store): CPU tensors of shape [M, lda] and [N, ldb].

    The logical operands are ``A_store[:, :K]`` and ``B_store[:, :K]``; columns K
    and beyond (present only when lda/ldb exceed K) hold NaN.
    """
    dt = _dtype(dtype)
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    if lda < K or ldb < K:
        raise ValueError("leading dimension below K")
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    a = _draw((M, K), dist, "A", g).to(dt)
    b = _draw((N, K), dist, "B", g).to(dt)
    if lda > K:
        A = torch.full((M, lda), float("nan"), dtype=dt)
        A[:, :K] = a
    else:
        A = a
    if ldb > K:
        B = torch.full((N, ldb), float("nan"), dtype=dt)
        B[:, :K] = b
    else:
        B = b
    return A.contiguous(), B.contiguous()


def store(X, layout, ld=None):
    """Lay the logical operand X [rows, K] out in memory: "k" keeps it row-major
    ([rows][ld >= K]); "mn" stores its transpose ([K][ld >= rows]).  Padding
    columns hold NaN."""
    rows, K = X.shape
    if layout == "k":
        src, extent = X, K
    elif layout == "mn":
        src, extent = X.t(), rows
    else:
        raise ValueError("unknown layout %r" % (layout,))
    ld = extent if ld is None else ld
    if ld < extent:
        raise ValueError("leading dimension below the stored row length")
    out = torch.full((src.shape[0], ld), float("nan"), dtype=X.dtype)
    out[:, :extent] = src
    return out.contiguous()


def make_stored(M, N, K, layout_a="k", layout_b="k", dtype="bf16", dist="uniform", seed=0,
                lda=None, ldb=None):
    """make_operands' values (same seed, same bits), each operand laid out by
    store(): A as [M][lda] or [K][lda], B as [N][ldb] or [K][ldb]."""
    A, B = make_operands(M, N, K, dtype, dist, seed)
    return store(A, layout_a, lda), store(B, layout_b, ldb)


FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}
_FP8_TORCH = {"e4m3": "float8_e4m3fn", "e5m2": "float8_e5m2"}
FP8_NAN = 0x7F            # a NaN code in both formats, used for padding


def _fp8_codes(x, fmt):
    """RNE FP8 codes (uint8) of float32 values already inside the format's range."""
    return x.to(getattr(torch, _FP8_TORCH[fmt])).view(torch.uint8)


def _quantize(x, fmt, mode, block_rows):
    """(codes, scales) of float32 values: a scale per tensor or per
    (block_rows x 128) block equal to the block's largest magnitude over the
    format's largest finite value (1 for an all-zero block)."""
    fmax = FP8_MAX[fmt]
    if mode == "tensor":
        amax = float(x.abs().max()) if x.numel() else 0.0
        s = torch.tensor([amax / fmax if amax > 0 else 1.0], dtype=torch.float32)
        return _fp8_codes((x / s).clamp(-fmax, fmax), fmt), s
    rows, K = x.shape
    nrb, nkb = -(-rows // block_rows), -(-K // 128)
    xp = torch.zeros((nrb * block_rows, nkb * 128), dtype=torch.float32)
    xp[:rows, :K] = x
    amax = xp.abs().reshape(nrb, block_rows, nkb, 128).amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / fmax, torch.ones_like(amax))
    q = xp / s.repeat_interleave(block_rows, 0).repeat_interleave(128, 1)
    return _fp8_codes(q[:rows, :K].clamp(-fmax, fmax), fmt), s.contiguous()


def _pow2_scales(mode, rows, K, block_rows, salt):
    """Powers of two from 2^-1 to 2^1, different in neighbouring blocks (small
    enough that every FP32 partial of a K <= 1024 product stays exact)."""
    if mode == "tensor":
        return torch.tensor([2.0 ** (salt % 3 - 1)], dtype=torch.float32)
    nrb, nkb = -(-rows // block_rows), -(-K // 128)
    e = (torch.arange(nrb)[:, None] * 2 + torch.arange(nkb)[None, :] + salt) % 3 - 1
    return torch.exp2(e.to(torch.float32))


def make_fp8_operands(M, N, K, fmt_a="e4m3", fmt_b="e4m3", dist="uniform", seed=0,
                      mode="tensor", block_m=1, lda=None, ldb=None):
    """(A codes [M, lda], B codes [N, ldb], scales of A, scales of B).

    Codes are uint8 tensors of OCP FP8 values; padding columns hold a NaN code.
    Scales are float32: one value each ("tensor"), or [ceil(M / block_m)][ceil(K / 128)]
    for A and [ceil(N / 128)][ceil(K / 128)] for B ("block").
      * "uniform" / "llm": make_operands' float32 draws quantized with
        amax scaling per tensor or per block (the recipe of blockwise FP8);
      * "int3": integers in {-3, ..., 3} with power-of-two scales, so that every
        partial sum is exact in FP32.
    """
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    if lda < K or ldb < K:
        raise ValueError("leading dimension below K")
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    if dist == "int3":
        xa = torch.randint(-3, 4, (M, K), generator=g, dtype=torch.int64).to(torch.float32)
        xb = torch.randint(-3, 4, (N, K), generator=g, dtype=torch.int64).to(torch.float32)
        qa, sa = _fp8_codes(xa, fmt_a), _pow2_scales(mode, M, K, block_m, 1)
        qb, sb = _fp8_codes(xb, fmt_b), _pow2_scales(mode, N, K, 128, 3)
    else:
        xa = _draw((M, K), dist, "A", g)
        xb = _draw((N, K), dist, "B", g)
        qa, sa = _quantize(xa, fmt_a, mode, block_m)
        qb, sb = _quantize(xb, fmt_b, mode, 128)
    A = torch.full((M, lda), FP8_NAN, dtype=torch.uint8)
    A[:, :K] = qa
    B = torch.full((N, ldb), FP8_NAN, dtype=torch.uint8)
    B[:, :K] = qb
    return A.contiguous(), B.contiguous(), sa.contiguous(), sb.contiguous()


def rotation_sets(M, N, K, dtype, dist, seed, count):
    """`count` independent operand pairs (seeds seed, seed+1, ...) for cold-cache timing."""
    return [make_operands(M, N, K, dtype, dist, seed + i) for i in range(count)]
