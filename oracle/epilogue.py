"""CPU oracle for the fused GEMM epilogue -- test infrastructure.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU library never does.

What it computes (the plain definition, elementwise, in binary64):

    D[i, j] = act( alpha * C_ref[i, j] + beta * C_old[i, j] + bias )

- "CUTLASS Deep Dive: From CuTe Layouts to Blackwell tcgen05", the Tutorial 01
  and 05 epilogues and "Epilogue Visitor Trees (EVT)": the epilogue scales the
  accumulator by alpha and adds beta times the existing C (axpby); the
  "Classic Fused Epilogue: Bias + ReLU" passage adds a bias and takes
  max(0, .) as the tile is written back.
- C_ref is the exact product from ``oracle.gemm_nt`` (binary64) and C_old the
  prior contents of C in the output format, decoded exactly.
- bias is an FP32 vector along the output columns (one value per n, the
  per-output-feature bias of a linear layer whose weights are the rows of B)
  or along the output rows (one value per m); the pages' example names a
  per-row bias in a column-major library convention, so both are offered.
- act is "none", "relu" (max(0, x), as printed) or "gelu", which the pages
  name only as "activation functions": read here as the exact form
  x * Phi(x) = x / 2 * (1 + erf(x / sqrt 2)).

Parity pins: tests/test_oracle_pins.py (identity, closed forms with exact
small values, both bias orientations on a non-square case, ReLU signs, and
GELU against printed standard-normal table values of Phi).
"""
from __future__ import annotations

import math

import numpy as np

ACTIVATIONS = ("none", "relu", "gelu")
BIAS_ALONG = ("none", "n", "m")


def _gelu(x: np.ndarray) -> np.ndarray:
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def apply(C_ref, C_old=None, alpha=1.0, beta=0.0, bias=None, bias_along="none", act="none"):
    """D (binary64) from the exact product C_ref (M x N, binary64).

    C_old: the prior output values as binary64 (M x N), required when beta != 0.
    bias: FP32 values (length N for bias_along="n", M for "m").
    """
    C_ref = np.asarray(C_ref, dtype=np.float64)
    if act not in ACTIVATIONS:
        raise ValueError("unknown activation %r" % (act,))
    if bias_along not in BIAS_ALONG:
        raise ValueError("unknown bias orientation %r" % (bias_along,))
    x = float(alpha) * C_ref
    if beta != 0.0:
        if C_old is None:
            raise ValueError("beta != 0 needs the prior output values")
        x = x + float(beta) * np.asarray(C_old, dtype=np.float64)
    if bias_along != "none":
        b = np.asarray(bias, dtype=np.float32).astype(np.float64)
        M, N = C_ref.shape
        if bias_along == "n":
            if b.shape != (N,):
                raise ValueError("bias along n needs N values")
            x = x + b[None, :]
        else:
            if b.shape != (M,):
                raise ValueError("bias along m needs M values")
            x = x + b[:, None]
    if act == "relu":
        x = np.maximum(x, 0.0)
    elif act == "gelu":
        x = _gelu(x)
    return x


def scale_of(S, C_old=None, alpha=1.0, beta=0.0, bias=None, bias_along="none"):
    """Magnitude terms the acceptance bound is stated in: (|alpha| S, the
    magnitude of the FP32 terms added after the sum)."""
    S = np.asarray(S, dtype=np.float64)
    t = np.zeros_like(S)
    if beta != 0.0:
        t = t + abs(float(beta)) * np.abs(np.asarray(C_old, dtype=np.float64))
    if bias_along != "none":
        b = np.abs(np.asarray(bias, dtype=np.float32).astype(np.float64))
        t = t + (b[None, :] if bias_along == "n" else b[:, None])
    return abs(float(alpha)) * S, t
