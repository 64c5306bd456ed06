"""ctypes binding of the C ABI in include/gemm_nt.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgemm_nt.so")

GEMM_BF16, GEMM_FP16, GEMM_FP32 = 0, 1, 2
GEMM_FP8_E4M3, GEMM_FP8_E5M2 = 3, 4
FP8_FORMATS = {"e4m3": GEMM_FP8_E4M3, "e5m2": GEMM_FP8_E5M2}
GEMM_SCALE_TENSOR, GEMM_SCALE_BLOCK = 0, 1
SCALE_MODES = {"tensor": GEMM_SCALE_TENSOR, "block": GEMM_SCALE_BLOCK}
GEMM_OK = 0
GEMM_ERR_INVALID_ARG, GEMM_ERR_UNSUPPORTED, GEMM_ERR_MISALIGNED = 1, 2, 3
STATUS = {0: "GEMM_OK", 1: "GEMM_ERR_INVALID_ARG", 2: "GEMM_ERR_UNSUPPORTED",
          3: "GEMM_ERR_MISALIGNED", 4: "GEMM_ERR_ALLOC", 5: "GEMM_ERR_HIP"}

# Every symbol include/gemm_nt.h declares.
EXPORTS = ("gemm_create", "gemm_run", "gemm_run_ex", "gemm_run_layout", "gemm_run_fp8",
           "gemm_run_grouped", "gemm_run_grouped_fp8", "gemm_destroy", "gemm_validate",
           "gemm_plan", "gemm_status_string", "gemm_run_noalloc")


class GemmError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__("%s%s" % (STATUS.get(status, "status %d" % status),
                                   (": " + what) if what else ""))


class GemmPlan(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int), ("block_n", ctypes.c_int), ("block_k", ctypes.c_int),
                ("waves", ctypes.c_int), ("stages", ctypes.c_int), ("splits", ctypes.c_int),
                ("lds_bytes", ctypes.c_int),
                ("tiles", ctypes.c_int64), ("workgroups", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("name", ctypes.c_char * 48),
                ("streamk", ctypes.c_int), ("inreduce", ctypes.c_int)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["name"] = self.name.decode()
        return d


class GemmEpilogue(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("bias", ctypes.c_void_p),
                ("bias_along", ctypes.c_int), ("activation", ctypes.c_int)]


class GemmFP8Scales(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("block_m", ctypes.c_int)]


class GemmGroupProblem(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64),
                ("ldc", ctypes.c_int64)]


class GemmGroupProblemFP8(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("scale_a", ctypes.c_void_p),
                ("scale_b", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64),
                ("ldc", ctypes.c_int64)]


BIAS_ALONG = {"none": 0, "n": 1, "m": 2}
GEMM_K_MAJOR, GEMM_MN_MAJOR = 0, 1
ACTIVATION = {"none": 0, "relu": 1, "gelu": 2}

_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgemm_nt.so is not built; run `python -m dense_gemm_nt_amd.build` "
                           "or __graft_entry__.build() first")
    # torch first: it carries its own copy of the HIP runtime, and the library
    # must bind to the one torch's memory and streams come from (loaded before
    # torch, it bound the system copy and gemm_create returned GEMM_ERR_HIP)
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.gemm_create.argtypes = [ctypes.POINTER(vp)]
    L.gemm_create.restype = ci
    L.gemm_destroy.argtypes = [vp]
    L.gemm_destroy.restype = ci
    L.gemm_run.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, ci, vp]
    L.gemm_run.restype = ci
    L.gemm_run_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, ci, vp]
    L.gemm_run_noalloc.restype = ci
    L.gemm_run_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, ci,
                              ctypes.POINTER(GemmEpilogue), vp]
    L.gemm_run_ex.restype = ci
    L.gemm_run_layout.argtypes = [vp, ci, ci, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, ci,
                                  ctypes.POINTER(GemmEpilogue), vp]
    L.gemm_run_layout.restype = ci
    L.gemm_run_fp8.argtypes = [vp, ci, ci, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci,
                               ctypes.POINTER(GemmFP8Scales), ctypes.POINTER(GemmEpilogue), vp]
    L.gemm_run_fp8.restype = ci
    L.gemm_run_grouped.argtypes = [vp, ctypes.POINTER(GemmGroupProblem), ci, ci, ci,
                                   ctypes.POINTER(GemmEpilogue), vp]
    L.gemm_run_grouped.restype = ci
    L.gemm_run_grouped_fp8.argtypes = [vp, ci, ci, ctypes.POINTER(GemmGroupProblemFP8), ci, ci, ci,
                                       ci, ctypes.POINTER(GemmEpilogue), vp]
    L.gemm_run_grouped_fp8.restype = ci
    L.gemm_validate.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, ci]
    L.gemm_validate.restype = ci
    L.gemm_plan.argtypes = [i64, i64, i64, ci, ci, ctypes.POINTER(GemmPlan)]
    L.gemm_plan.restype = ci
    L.gemm_status_string.argtypes = [ci]
    L.gemm_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def check(status, what=""):
    if status != GEMM_OK:
        raise GemmError(status, what)


def gemm_create():
    h = ctypes.c_void_p()
    check(lib().gemm_create(ctypes.byref(h)), "gemm_create")
    return h


def gemm_destroy(h):
    check(lib().gemm_destroy(h), "gemm_destroy")


def gemm_run(h, A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype, stream):
    """Raw entry point: A, B, C and stream are integer device addresses / a hipStream_t."""
    return lib().gemm_run(h, A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype, stream)


def gemm_run_ex(h, A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype, epi, stream):
    """Raw entry point with a fused epilogue (a GemmEpilogue or None)."""
    return lib().gemm_run_ex(h, A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype,
                             ctypes.byref(epi) if epi is not None else None, stream)


def gemm_run_layout(h, layout_a, layout_b, A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype,
                    epi, stream):
    """Raw entry point for any operand layouts (GEMM_K_MAJOR / GEMM_MN_MAJOR each)."""
    return lib().gemm_run_layout(h, layout_a, layout_b, A, B, C, M, N, K, lda, ldb, ldc, in_dtype,
                                 out_dtype, ctypes.byref(epi) if epi is not None else None, stream)


def gemm_run_fp8(h, a_dtype, b_dtype, A, B, C, M, N, K, lda, ldb, ldc, out_dtype, scales, epi,
                 stream):
    """Raw FP8 entry point: `scales` a GemmFP8Scales (or None), `epi` a GemmEpilogue or None."""
    return lib().gemm_run_fp8(h, a_dtype, b_dtype, A, B, C, M, N, K, lda, ldb, ldc, out_dtype,
                              ctypes.byref(scales) if scales is not None else None,
                              ctypes.byref(epi) if epi is not None else None, stream)


def gemm_run_grouped(h, problems, in_dtype, out_dtype, epi, stream):
    """Raw grouped entry point: `problems` a list of GemmGroupProblem."""
    arr = (GemmGroupProblem * len(problems))(*problems)
    return lib().gemm_run_grouped(h, arr if problems else None, len(problems), in_dtype,
                                  out_dtype, ctypes.byref(epi) if epi is not None else None,
                                  stream)


def gemm_run_grouped_fp8(h, a_dtype, b_dtype, problems, out_dtype, scale_mode, block_m, epi,
                         stream):
    """Raw grouped FP8 entry point: `problems` a list of GemmGroupProblemFP8."""
    arr = (GemmGroupProblemFP8 * len(problems))(*problems)
    return lib().gemm_run_grouped_fp8(h, a_dtype, b_dtype, arr if problems else None,
                                      len(problems), out_dtype, SCALE_MODES[scale_mode],
                                      int(block_m), ctypes.byref(epi) if epi is not None else None,
                                      stream)


def fp8_scales(mode, a, b, block_m=1):
    """A GemmFP8Scales; `a`, `b` are integer device addresses of FP32 scales."""
    if mode not in SCALE_MODES:
        raise ValueError("mode must be one of %s" % sorted(SCALE_MODES))
    return GemmFP8Scales(SCALE_MODES[mode], a or None, b or None, int(block_m))


def epilogue(alpha=1.0, beta=0.0, bias=0, bias_along="none", activation="none"):
    """A GemmEpilogue; `bias` is an integer device address (0 for none)."""
    if bias_along not in BIAS_ALONG:
        raise ValueError("bias_along must be one of %s" % sorted(BIAS_ALONG))
    if activation not in ACTIVATION:
        raise ValueError("activation must be one of %s" % sorted(ACTIVATION))
    return GemmEpilogue(float(alpha), float(beta), bias or None, BIAS_ALONG[bias_along],
                        ACTIVATION[activation])


def gemm_validate(A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype):
    return lib().gemm_validate(A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype)


def gemm_plan(M, N, K, in_dtype=GEMM_BF16, out_dtype=GEMM_BF16):
    p = GemmPlan()
    check(lib().gemm_plan(M, N, K, in_dtype, out_dtype, ctypes.byref(p)), "gemm_plan")
    return p.as_dict()


def gemm_status_string(s):
    return lib().gemm_status_string(s).decode()
