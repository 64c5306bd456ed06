"""CPU oracle for the NT GEMM ``C[M,N] = A[M,K] . B[N,K]^T`` -- test infrastructure.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it and the
two share no code: the oracle is ``gemm_oracle.c`` (a naive binary64 triple loop,
see its header for the passages it follows) built with gcc, plus this ctypes
loader.  Inputs are the raw 16-bit codes of A and B (numpy ``uint16`` arrays);
outputs are binary64 numpy arrays.

Parity pins for every function here live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "libgemm_oracle.so")

BF16 = 0
FP16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) into this folder."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = ctypes.c_double
    lib.oracle_decode_fp16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_fp16.restype = ctypes.c_double
    lib.oracle_encode_bf16.argtypes = [ctypes.c_double]
    lib.oracle_encode_bf16.restype = ctypes.c_uint16
    lib.oracle_encode_fp16.argtypes = [ctypes.c_double]
    lib.oracle_encode_fp16.restype = ctypes.c_uint16
    lib.oracle_gemm_nt.argtypes = [u16p, u16p, i64, i64, i64, i64, i64, ctypes.c_int, f64p, f64p]
    lib.oracle_gemm_nt.restype = ctypes.c_int
    lib.oracle_gemm_nt_rows.argtypes = [u16p, u16p, i64, i64, i64, i64, i64, ctypes.c_int,
                                        i64p, i64, f64p, f64p]
    lib.oracle_gemm_nt_rows.restype = ctypes.c_int
    lib.oracle_gemm_nt_points.argtypes = [u16p, u16p, i64, i64, i64, i64, i64, ctypes.c_int,
                                          i64p, i64p, i64, f64p, f64p]
    lib.oracle_gemm_nt_points.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _codes(x) -> np.ndarray:
    """A 2-D array of 16-bit codes: numpy uint16, or a torch bf16/fp16 tensor (CPU)."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("oracle expects uint16 codes")
        return x
    import torch  # only for the view of a 16-bit tensor's bits
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("oracle expects bf16/fp16 tensors")
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _operand(x, rows, K):
    """(pointer, leading dimension) of a row-major operand whose first K columns are read."""
    c = _codes(x)
    if c.ndim != 2 or c.shape[0] != rows or c.shape[1] < K:
        raise ValueError("operand shape %r does not cover %d x %d" % (c.shape, rows, K))
    if c.strides[1] != 2:
        c = np.ascontiguousarray(c)
    ld = c.strides[0] // 2
    if c.strides[0] % 2 or ld < K:
        c = np.ascontiguousarray(c)
        ld = c.shape[1]
    return c, ld


def dtype_code(name) -> int:
    name = str(name).replace("torch.", "")
    if name in ("bf16", "bfloat16"):
        return BF16
    if name in ("fp16", "f16", "float16", "half"):
        return FP16
    raise ValueError("unknown input format %r" % name)


def gemm_nt(A, B, K=None, in_dtype="bf16", with_abs=True):
    """C_ref, S for the whole product.  A: M x (>=K) codes, B: N x (>=K) codes."""
    lib = _load()
    Ac = _codes(A)
    Bc = _codes(B)
    M, N = Ac.shape[0], Bc.shape[0]
    K = Ac.shape[1] if K is None else K
    a, lda = _operand(Ac, M, K)
    b, ldb = _operand(Bc, N, K)
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64) if with_abs else None
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_gemm_nt(a.ctypes.data_as(u16p), b.ctypes.data_as(u16p), M, N, K, lda, ldb,
                            dtype_code(in_dtype), C.ctypes.data_as(f64p),
                            S.ctypes.data_as(f64p) if S is not None else None)
    if rc != 0:
        raise ValueError("oracle_gemm_nt rejected its arguments")
    return C, S


def gemm_nt_rows(A, B, rows, K=None, in_dtype="bf16"):
    """C_ref, S restricted to the given rows of the product (len(rows) x N)."""
    lib = _load()
    Ac = _codes(A)
    Bc = _codes(B)
    M, N = Ac.shape[0], Bc.shape[0]
    K = Ac.shape[1] if K is None else K
    a, lda = _operand(Ac, M, K)
    b, ldb = _operand(Bc, N, K)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    C = np.empty((r.size, N), dtype=np.float64)
    S = np.empty((r.size, N), dtype=np.float64)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    rc = lib.oracle_gemm_nt_rows(a.ctypes.data_as(u16p), b.ctypes.data_as(u16p), M, N, K, lda,
                                 ldb, dtype_code(in_dtype), r.ctypes.data_as(i64p), r.size,
                                 C.ctypes.data_as(f64p), S.ctypes.data_as(f64p))
    if rc != 0:
        raise ValueError("oracle_gemm_nt_rows rejected its arguments")
    return C, S


def gemm_nt_points(A, B, ii, jj, K=None, in_dtype="bf16"):
    """C_ref[p], S[p] at output coordinates (ii[p], jj[p])."""
    lib = _load()
    Ac = _codes(A)
    Bc = _codes(B)
    M, N = Ac.shape[0], Bc.shape[0]
    K = Ac.shape[1] if K is None else K
    a, lda = _operand(Ac, M, K)
    b, ldb = _operand(Bc, N, K)
    ii = np.ascontiguousarray(np.asarray(ii, dtype=np.int64))
    jj = np.ascontiguousarray(np.asarray(jj, dtype=np.int64))
    if ii.shape != jj.shape:
        raise ValueError("ii and jj differ in length")
    C = np.empty(ii.size, dtype=np.float64)
    S = np.empty(ii.size, dtype=np.float64)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    rc = lib.oracle_gemm_nt_points(a.ctypes.data_as(u16p), b.ctypes.data_as(u16p), M, N, K,
                                   lda, ldb, dtype_code(in_dtype), ii.ctypes.data_as(i64p),
                                   jj.ctypes.data_as(i64p), ii.size, C.ctypes.data_as(f64p),
                                   S.ctypes.data_as(f64p))
    if rc != 0:
        raise ValueError("oracle_gemm_nt_points rejected its arguments")
    return C, S


LAYOUTS = ("k", "mn")


def logical_operand(X, layout, rows=None, K=None) -> np.ndarray:
    """The [rows, K] operand (codes) that a stored array X holds.

    Page "Steps for Writing a Speed-of-Light GEMM kernel: Part 1", the CuTe
    introduction ("A tensor is storage plus a layout"): a layout maps the
    logical coordinate to a storage offset, (m, k) -> m * ld + k for a
    row-major (K-major) operand.  An MN-major operand stores the same matrix
    with the roles of the two indices exchanged, (m, k) -> k * ld + m, i.e. X is
    [K][>= rows] and the operand is its transpose.  Page "Optimizing GEMMs using
    tcgen05 - Part 1" ("What I am measuring") multiplies a row-major A [M, K] by
    a row-major B [K, N]: here that B is the N-major operand of A . B^T.
    """
    c = _codes(X)
    if c.ndim != 2:
        raise ValueError("operand must be 2-D")
    if layout == "k":
        rows = c.shape[0] if rows is None else rows
        K = c.shape[1] if K is None else K
        if c.shape[0] < rows or c.shape[1] < K:
            raise ValueError("stored %r does not cover %d x %d" % (c.shape, rows, K))
        return c[:rows, :K]
    if layout == "mn":
        rows = c.shape[1] if rows is None else rows
        K = c.shape[0] if K is None else K
        if c.shape[1] < rows or c.shape[0] < K:
            raise ValueError("stored %r does not cover %d x %d (transposed)" % (c.shape, K, rows))
        return np.ascontiguousarray(c[:K, :rows].T)
    raise ValueError("unknown layout %r" % (layout,))


def gemm(A, B, layout_a="k", layout_b="k", K=None, in_dtype="bf16", with_abs=True):
    """C_ref, S of sum_k a(i,k) b(j,k) with each operand read through its layout
    (logical_operand); (k, k) is gemm_nt."""
    a = logical_operand(A, layout_a, K=K)
    b = logical_operand(B, layout_b, K=K)
    if a.shape[1] != b.shape[1]:
        raise ValueError("inner dimensions differ: %d vs %d" % (a.shape[1], b.shape[1]))
    return gemm_nt(a, b, in_dtype=in_dtype, with_abs=with_abs)


def gemm_points(A, B, ii, jj, layout_a="k", layout_b="k", K=None, in_dtype="bf16"):
    """C_ref[p], S[p] at (ii[p], jj[p]) of the product gemm() defines."""
    a = logical_operand(A, layout_a, K=K)
    b = logical_operand(B, layout_b, K=K)
    if a.shape[1] != b.shape[1]:
        raise ValueError("inner dimensions differ: %d vs %d" % (a.shape[1], b.shape[1]))
    return gemm_nt_points(a, b, ii, jj, in_dtype=in_dtype)


def gemm_grouped(problems, in_dtype="bf16"):
    """[(C_ref_g, S_g)] for a list of problems (A_g, B_g, K_g): one independent
    NT product per group.

    "CUTLASS Deep Dive: From CuTe Layouts to Blackwell tcgen05", "Grouped GEMM
    -- MoE's workhorse": a batch of GEMMs of different shapes (one per expert)
    computed in one launch; what each group computes is the plain product of
    its own operands, so the oracle is that product per group.
    """
    return [gemm_nt(A, B, K=K, in_dtype=in_dtype) for (A, B, K) in problems]


def decode(codes, in_dtype="bf16") -> np.ndarray:
    """Exact binary64 values of an array of 16-bit codes."""
    lib = _load()
    f = lib.oracle_decode_bf16 if dtype_code(in_dtype) == BF16 else lib.oracle_decode_fp16
    c = np.asarray(codes, dtype=np.uint16)
    return np.array([f(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def encode(values, out_dtype="bf16") -> np.ndarray:
    """Round-to-nearest-even 16-bit codes of binary64 values."""
    lib = _load()
    f = lib.oracle_encode_bf16 if dtype_code(out_dtype) == BF16 else lib.oracle_encode_fp16
    v = np.asarray(values, dtype=np.float64)
    return np.array([f(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)


def num_threads() -> int:
    return int(_load().oracle_num_threads())
