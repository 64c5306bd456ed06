"""MI355X (gfx950) NT GEMM: C[M,N] = A[M,K] . B[N,K]^T with BF16/FP16 inputs (any
operand layout, fused epilogue) and FP8 inputs with per-tensor or blockwise scales.

The computation runs in the HIP library ``libgemm_nt.so`` (C ABI in
``include/gemm_nt.h``); this package only marshals arguments.  PyTorch provides
device memory and streams.  There is no CPU fallback: without the built library
every call raises.
"""
from ._lib import (GEMM_BF16, GEMM_FP16, GEMM_FP32, GEMM_FP8_E4M3, GEMM_FP8_E5M2, GemmError,
                   gemm_create, gemm_destroy, gemm_plan, gemm_run, gemm_status_string,
                   gemm_validate)
from .api import Gemm, default_handle, gemm_fp8, gemm_grouped, gemm_nt

__all__ = ["GEMM_BF16", "GEMM_FP16", "GEMM_FP32", "GEMM_FP8_E4M3", "GEMM_FP8_E5M2", "GemmError",
           "Gemm", "default_handle", "gemm_fp8", "gemm_grouped", "gemm_nt", "gemm_create", "gemm_destroy",
           "gemm_plan", "gemm_run", "gemm_status_string", "gemm_validate"]
