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


def _operand(X, rows, K):
    """(layout, leading dimension) of a [rows, K] operand view: K-major when its
    K stride is 1, MN-major (a transposed view of a [K, rows] array) when its row
    stride is 1."""
    if K == 0 or rows == 0:
        return _lib.GEMM_K_MAJOR, max(K, 1)
    if X.stride(1) == 1 and (rows == 1 or X.stride(0) >= K):
        return _lib.GEMM_K_MAJOR, X.stride(0) if rows > 1 else max(K, X.stride(0))
    if X.stride(0) == 1 and (K == 1 or X.stride(1) >= rows):
        return _lib.GEMM_MN_MAJOR, X.stride(1) if K > 1 else max(rows, X.stride(1))
    raise ValueError("operand strides %s are neither K-major nor MN-major" % (tuple(X.stride()),))


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

    def run_raw_ex(self, A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype, epi, stream):
        st = _lib.gemm_run_ex(self._h, A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype, epi,
                              stream)
        _lib.check(st, "gemm_run_ex(M=%d, N=%d, K=%d)" % (M, N, K))

    def run_raw_layout(self, layout_a, layout_b, A, B, C, M, N, K, lda, ldb, ldc, in_dtype,
                       out_dtype, epi, stream):
        st = _lib.gemm_run_layout(self._h, layout_a, layout_b, A, B, C, M, N, K, lda, ldb, ldc,
                                  in_dtype, out_dtype, epi, stream)
        _lib.check(st, "gemm_run_layout(%d, %d, M=%d, N=%d, K=%d)" % (layout_a, layout_b, M, N, K))

    def run_raw_fp8(self, a_dtype, b_dtype, A, B, C, M, N, K, lda, ldb, ldc, out_dtype, scales,
                    epi, stream):
        st = _lib.gemm_run_fp8(self._h, a_dtype, b_dtype, A, B, C, M, N, K, lda, ldb, ldc,
                               out_dtype, scales, epi, stream)
        _lib.check(st, "gemm_run_fp8(M=%d, N=%d, K=%d)" % (M, N, K))

    def grouped(self, As, Bs, outs=None, out_dtype=None, stream=None, alpha=1.0, beta=0.0,
                biases=None, bias_along="n", activation="none"):
        """[C_g = act(alpha * A_g . B_g^T + beta * C_g_old + bias_g)] for lists of CUDA
        tensors A_g [M_g, K_g] and B_g [N_g, K_g] (one dtype, unit stride along K),
        in one launch.  `outs` (needed when beta != 0) and `biases` are lists too."""
        import torch
        G = len(As)
        if len(Bs) != G or (outs is not None and len(outs) != G) or \
                (biases is not None and len(biases) != G):
            raise ValueError("As, Bs, outs and biases must have one entry per group")
        if beta != 0.0 and outs is None:
            raise ValueError("beta != 0 reads the prior C: pass `outs`")
        if G == 0:
            return []
        dt = As[0].dtype
        dev = As[0].device
        probs, res = [], []
        for g in range(G):
            A, B = As[g], Bs[g]
            if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
                raise ValueError("group %d: A [M, K] and B [N, K] expected" % g)
            if A.dtype != dt or B.dtype != dt or A.device != dev or B.device != dev:
                raise TypeError("group %d: every operand must share dtype and device" % g)
            M, K = A.shape
            N = B.shape[0]
            if K > 0 and (A.stride(1) != 1 or B.stride(1) != 1):
                raise ValueError("group %d: operands need unit stride along K" % g)
            C = outs[g] if outs is not None else torch.empty(
                (M, N), dtype=out_dtype or dt, device=dev)
            if tuple(C.shape) != (M, N) or (N > 0 and C.stride(1) != 1):
                raise ValueError("group %d: out must be [M, N] with unit column stride" % g)
            bias = None
            if biases is not None and biases[g] is not None:
                bias = biases[g]
                want = N if bias_along == "n" else M
                if bias.dtype != torch.float32 or bias.numel() != want or bias.stride(0) != 1:
                    raise ValueError("group %d: bias must be %d contiguous float32 values"
                                     % (g, want))
            res.append(C)
            probs.append(_lib.GemmGroupProblem(
                A.data_ptr(), B.data_ptr(), C.data_ptr(), bias.data_ptr() if bias is not None
                else None, M, N, K, A.stride(0) if M > 1 else max(K, A.stride(0)),
                B.stride(0) if N > 1 else max(K, B.stride(0)),
                C.stride(0) if M > 1 else max(N, C.stride(0))))
        out_dt = res[0].dtype
        if any(c.dtype != out_dt for c in res):
            raise TypeError("every output must share one dtype")
        with_bias = biases is not None and any(b is not None for b in biases)
        epi = None
        if not (alpha == 1.0 and beta == 0.0 and not with_bias and activation == "none"):
            epi = _lib.epilogue(alpha, beta, 0, bias_along if with_bias else "none", activation)
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        st = _lib.gemm_run_grouped(self._h, probs, _code(dt), _code(out_dt), epi, stream)
        _lib.check(st, "gemm_run_grouped(%d groups)" % G)
        return res

    def fp8(self, A, B, scale_a, scale_b, fmt_a="e4m3", fmt_b="e4m3", block_m=None, out=None,
            out_dtype=None, stream=None, alpha=1.0, beta=0.0, bias=None, bias_along="n",
            activation="none"):
        """C = act(alpha * sum_k sa a sb b + beta * C_old + bias) for FP8 CUDA tensors
        A [M, K] and B [N, K] (uint8 codes or torch float8, unit stride along K).
        scale_a / scale_b: float32 CUDA tensors with one value each (per tensor) or
        [ceil(M / block_m), ceil(K / 128)] and [ceil(N / 128), ceil(K / 128)]
        (blockwise; block_m 1 or 128, inferred from scale_a's shape when None)."""
        import torch
        if A.dim() != 2 or B.dim() != 2:
            raise ValueError("A and B must be 2-D")
        if beta != 0.0 and out is None:
            raise ValueError("beta != 0 reads the prior C: pass it as `out`")
        M, K = A.shape
        N, K2 = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
        if A.element_size() != 1 or B.element_size() != 1:
            raise TypeError("A and B must hold 8-bit codes")
        if K > 0 and (A.stride(1) != 1 or B.stride(1) != 1):
            raise ValueError("FP8 operands need unit stride along K")
        for sc in (scale_a, scale_b):
            if sc.dtype != torch.float32 or not sc.is_contiguous() or sc.device != A.device:
                raise ValueError("scales must be contiguous float32 tensors on %s" % A.device)
        nkb = -(-K // 128)
        if scale_a.numel() == 1 and scale_b.numel() == 1 and block_m is None:
            mode, block_m = "tensor", 1
        else:
            mode = "block"
            if block_m is None:
                block_m = 1 if scale_a.shape[0] == M else 128
            if tuple(scale_a.shape) != (-(-M // block_m), nkb) or \
                    tuple(scale_b.shape) != (-(-N // 128), nkb):
                raise ValueError("blockwise scales must be [%d, %d] and [%d, %d]"
                                 % (-(-M // block_m), nkb, -(-N // 128), nkb))
        if out is None:
            out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=A.device)
        if out.dim() != 2 or tuple(out.shape) != (M, N) or (N > 0 and out.stride(1) != 1):
            raise ValueError("out must be [M, N] with unit column stride")
        lda = A.stride(0) if M > 1 else max(K, A.stride(0))
        ldb = B.stride(0) if N > 1 else max(K, B.stride(0))
        ldc = out.stride(0) if M > 1 else max(N, out.stride(0))
        if stream is None:
            stream = torch.cuda.current_stream(A.device).cuda_stream
        epi = None
        if not (alpha == 1.0 and beta == 0.0 and bias is None and activation == "none"):
            epi = _lib.epilogue(alpha, beta, bias.data_ptr() if bias is not None else 0,
                                bias_along if bias is not None else "none", activation)
        scales = _lib.fp8_scales(mode, scale_a.data_ptr(), scale_b.data_ptr(), block_m)
        self.run_raw_fp8(_lib.FP8_FORMATS[fmt_a], _lib.FP8_FORMATS[fmt_b], A.data_ptr(),
                         B.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldc, _code(out.dtype),
                         scales, epi, stream)
        return out

    def __call__(self, A, B, out=None, out_dtype=None, stream=None, alpha=1.0, beta=0.0,
                 bias=None, bias_along="n", activation="none"):
        """C = act(alpha * A . B^T + beta * C_old + bias) for CUDA tensors A [M, K] and
        B [N, K].  Each operand is K-major (unit stride along K) or MN-major (unit
        stride along its rows: e.g. B = W.t() for a row-major W [K, N]).  beta != 0
        needs `out` holding C_old; `bias` is a float32 CUDA tensor of N values
        (bias_along="n") or M values ("m")."""
        import torch
        if A.dim() != 2 or B.dim() != 2:
            raise ValueError("A and B must be 2-D")
        if beta != 0.0 and out is None:
            raise ValueError("beta != 0 reads the prior C: pass it as `out`")
        M, K = A.shape
        N, K2 = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
        if A.dtype != B.dtype:
            raise TypeError("A and B must share a dtype")
        la, lda = _operand(A, M, K)
        lb, ldb = _operand(B, N, K)
        if out is None:
            out_dtype = A.dtype if out_dtype is None else out_dtype
            out = torch.empty((M, N), dtype=out_dtype, device=A.device)
        if out.dim() != 2 or tuple(out.shape) != (M, N) or (N > 0 and out.stride(1) != 1):
            raise ValueError("out must be [M, N] with unit column stride")
        ldc = out.stride(0) if M > 1 else max(N, out.stride(0))
        if stream is None:
            stream = torch.cuda.current_stream(A.device).cuda_stream
        plain = alpha == 1.0 and beta == 0.0 and bias is None and activation == "none"
        nt = la == _lib.GEMM_K_MAJOR and lb == _lib.GEMM_K_MAJOR
        if plain and nt:
            self.run_raw(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldc,
                         _code(A.dtype), _code(out.dtype), stream)
            return out
        along = "none"
        if bias is not None:
            along = bias_along
            want = N if along == "n" else M
            if bias.dtype != torch.float32 or bias.dim() != 1 or bias.numel() != want \
                    or bias.stride(0) != 1 or bias.device != A.device:
                raise ValueError("bias must be a contiguous float32 vector of %d values on %s"
                                 % (want, A.device))
        epi = None if plain else _lib.epilogue(alpha, beta, bias.data_ptr() if bias is not None
                                               else 0, along, activation)
        if not nt:
            self.run_raw_layout(la, lb, A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, lda,
                                ldb, ldc, _code(A.dtype), _code(out.dtype), epi, stream)
            return out
        self.run_raw_ex(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldc,
                        _code(A.dtype), _code(out.dtype), epi, stream)
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


def gemm_grouped(As, Bs, **kw):
    """Grouped GEMM over lists of operands in one launch, with the per-device
    default handle (see Gemm.grouped)."""
    import torch
    with torch.cuda.device(As[0].device):
        return default_handle(As[0].device.index).grouped(As, Bs, **kw)


def gemm_fp8(A, B, scale_a, scale_b, **kw):
    """FP8 GEMM with per-tensor or blockwise scales on A's device with the
    per-device default handle (see Gemm.fp8)."""
    import torch
    with torch.cuda.device(A.device):
        return default_handle(A.device.index).fp8(A, B, scale_a, scale_b, **kw)


def gemm_nt(A, B, out=None, out_dtype=None, **epilogue):
    """C = A . B^T on A's device with the per-device default handle (current stream);
    keyword arguments alpha, beta, bias, bias_along, activation select the fused
    epilogue (see Gemm.__call__)."""
    import torch
    with torch.cuda.device(A.device):
        return default_handle(A.device.index)(A, B, out=out, out_dtype=out_dtype, **epilogue)
