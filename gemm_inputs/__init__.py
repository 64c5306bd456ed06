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


def rotation_sets(M, N, K, dtype, dist, seed, count):
    """`count` independent operand pairs (seeds seed, seed+1, ...) for cold-cache timing."""
    return [make_operands(M, N, K, dtype, dist, seed + i) for i in range(count)]
