"""Acceptance check of a GPU result against the oracle (binary64, on the host).

Bound, for every output element (i, j):
    |C - C_ref| <= 1e-3 * S + 1e-5                          (fp32 output)
    |C - C_ref| <= 1e-3 * S + 1e-5 + ulp_out(max(|C_ref|, |C|))   (bf16 / fp16 output)
with S = sum_k |a(i,k) b(j,k)| from the oracle.  The relative term covers FP32
accumulation in any order (at most about K/16 rounded additions of partial sums,
each within 2^-24 of the running magnitude, which stays below S); the absolute
term covers results that cancel to near zero; the ulp term covers the final
rounding to a 16-bit format, taken at the larger magnitude so a rounding across a
binade boundary is allowed.
"""
from __future__ import annotations

import numpy as np

REL = 1e-3
ABS = 1e-5


def ulp(x: np.ndarray, out_dtype: str) -> np.ndarray:
    """Spacing of the 16-bit output format at |x| (its subnormal spacing below the normal range)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    if out_dtype in ("fp32", "float32"):
        return np.zeros_like(ax)
    if out_dtype in ("bf16", "bfloat16"):
        emin, fbits = -126, 7
    elif out_dtype in ("fp16", "float16"):
        emin, fbits = -14, 10
    else:
        raise ValueError(out_dtype)
    with np.errstate(divide="ignore"):
        e = np.where(ax > 0, np.floor(np.log2(np.where(ax > 0, ax, 1.0))), emin)
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - fbits).astype(np.int64))


def check(C_gpu, C_ref, S, out_dtype, what=""):
    """Assert the bound; return (max |err|, worst err / bound)."""
    c = np.asarray(C_gpu, dtype=np.float64)
    r = np.asarray(C_ref, dtype=np.float64)
    s = np.asarray(S, dtype=np.float64)
    if c.shape != r.shape:
        raise AssertionError("%s: shape %r vs oracle %r" % (what, c.shape, r.shape))
    if not np.all(np.isfinite(c)):
        bad = np.argwhere(~np.isfinite(c))[:5]
        raise AssertionError("%s: non-finite output at %s" % (what, bad.tolist()))
    err = np.abs(c - r)
    bound = REL * s + ABS + ulp(np.maximum(np.abs(r), np.abs(c)), out_dtype)
    ratio = err / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(
            "%s: |C-C_ref| above bound at %s: gpu=%r ref=%r S=%r err=%r bound=%r (%d elements over)"
            % (what, tuple(int(i) for i in idx), c[idx], r[idx], s[idx], err[idx], bound[idx],
               int((ratio > 1.0).sum())))
    return (float(err.max()) if err.size else 0.0), worst


def check_epilogue(D_gpu, D_ref, aS, t, out_dtype, what=""):
    """Acceptance of a fused-epilogue result D = act(alpha acc + beta C_old + bias).

    aS = |alpha| S and t = |beta C_old| + |bias| (oracle.epilogue.scale_of).  The
    sum's own bound 1e-3 S + 1e-5 is scaled by |alpha| and by 1.2 (the largest
    slope of GELU is 1.13; ReLU's is 1); 2^-20 (|alpha| S + t) covers the FP32
    multiply-adds after the sum and the activation's evaluation; the output
    ulp covers the final rounding.
    """
    c = np.asarray(D_gpu, dtype=np.float64)
    r = np.asarray(D_ref, dtype=np.float64)
    if c.shape != r.shape:
        raise AssertionError("%s: shape %r vs oracle %r" % (what, c.shape, r.shape))
    if not np.all(np.isfinite(c)):
        bad = np.argwhere(~np.isfinite(c))[:5]
        raise AssertionError("%s: non-finite output at %s" % (what, bad.tolist()))
    aS = np.asarray(aS, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    err = np.abs(c - r)
    bound = 1.2 * (REL * aS + ABS) + 2.0 ** -20 * (aS + t) + \
        ulp(np.maximum(np.abs(r), np.abs(c)), out_dtype)
    ratio = err / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(
            "%s: |D-D_ref| above bound at %s: gpu=%r ref=%r err=%r bound=%r (%d elements over)"
            % (what, tuple(int(i) for i in idx), c[idx], r[idx], err[idx], bound[idx],
               int((ratio > 1.0).sum())))
    return (float(err.max()) if err.size else 0.0), worst
