"""Tensor-level wrapper over the C ABI: shapes and strides in, device pointers out."""
from __future__ import annotations

import threading

from . import _lib

_TORCH_CODES = {"torch.bfloat16": _lib.GEMM_BF16, "torch.float16": _lib.GEMM_FP16,
                "torch.float32": _lib.GEMM_FP32}


def _code(dtype) -> int:
    c = _TORCH_CODES.get(str(dtype))
    if c is None:
        raise TypeError("unsupported dtype %s" % dtype)
    return c


class Gemm:
    """A library handle (workspace owner) bound to the current device."""

    def __init__(self):
        self._h = _lib.gemm_create()

    def close(self):
        if self._h is not None:
            _lib.gemm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run_raw(self, A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype, stream):
        st = _lib.gemm_run(self._h, A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype, stream)
        _lib.check(st, "gemm_run(M=%d, N=%d, K=%d)" % (M, N, K))

    def __call__(self, A, B, out=None, out_dtype=None, stream=None):
        """C = A . B^T for CUDA tensors A [M, K] and B [N, K] (unit column stride)."""
        import torch
        if A.dim() != 2 or B.dim() != 2:
            raise ValueError("A and B must be 2-D")
        M, K = A.shape
        N, K2 = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
        if A.dtype != B.dtype:
            raise TypeError("A and B must share a dtype")
        if K > 0 and (A.stride(1) != 1 or B.stride(1) != 1):
            raise ValueError("A and B need unit stride along K")
        if out is None:
            out_dtype = A.dtype if out_dtype is None else out_dtype
            out = torch.empty((M, N), dtype=out_dtype, device=A.device)
        if out.dim() != 2 or tuple(out.shape) != (M, N) or (N > 0 and out.stride(1) != 1):
            raise ValueError("out must be [M, N] with unit column stride")
        lda = A.stride(0) if M > 1 else max(K, A.stride(0))
        ldb = B.stride(0) if N > 1 else max(K, B.stride(0))
        ldc = out.stride(0) if M > 1 else max(N, out.stride(0))
        if stream is None:
            stream = torch.cuda.current_stream(A.device).cuda_stream
        self.run_raw(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldc,
                     _code(A.dtype), _code(out.dtype), stream)
        return out


_handles = {}
_lock = threading.Lock()


def default_handle(device_index: int) -> Gemm:
    with _lock:
        h = _handles.get(device_index)
        if h is None:
            h = Gemm()
            _handles[device_index] = h
        return h


def gemm_nt(A, B, out=None, out_dtype=None):
    """C = A . B^T on A's device with the per-device default handle (current stream)."""
    import torch
    with torch.cuda.device(A.device):
        return default_handle(A.device.index)(A, B, out=out, out_dtype=out_dtype)
