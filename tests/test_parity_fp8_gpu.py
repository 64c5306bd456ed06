"""Parity of the FP8 GEMM (gemm_run_fp8, through the C ABI) with the oracle
(oracle/fp8.py) on the same seeded FP8 codes and scales.

Cases: both formats for each operand, per-tensor and blockwise scales (per row
and per 128 rows of A), ragged M, N and a K tail shorter than a scale block;
small integers with power-of-two scales (every FP32 partial exact, so the
comparison is bitwise) with and without split-K; zero scales; the decode
shape; the fused epilogue; the 4096^3 workload on sampled outputs; the torch
binding; the argument checks.
"""
import numpy as np
import pytest
import torch

from oracle import epilogue as oepi
from oracle import fp8 as ofp8
from dense_gemm_nt_amd import _lib
from gemm_inputs import make_fp8_operands
from tests.gpu_util import CODE, TORCH_DT, new_handle, say
from tests.tolerance import check, check_epilogue

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
FMT = {"e4m3": _lib.GEMM_FP8_E4M3, "e5m2": _lib.GEMM_FP8_E5M2}


def _run(h, A, B, sa, sb, K, fa, fb, mode, block_m, out_dt, epi=None, C_old=None, ldc=None):
    M, lda = A.shape
    N, ldb = B.shape
    ldc = N if ldc is None else ldc
    Ad, Bd, sad, sbd = A.to(DEV), B.to(DEV), sa.to(DEV), sb.to(DEV)
    if C_old is None:
        Cd = torch.full((max(M, 1), max(ldc, 1)), float("nan"), dtype=TORCH_DT[out_dt], device=DEV)
    else:
        Cd = C_old.to(DEV).clone()
    scales = _lib.fp8_scales(mode, sad.data_ptr(), sbd.data_ptr(), block_m)
    s = torch.cuda.current_stream(DEV)
    h.run_raw_fp8(FMT[fa], FMT[fb], Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), M, N, K, lda, ldb,
                  ldc, CODE[out_dt], scales, epi, s.cuda_stream)
    s.synchronize()
    return Cd[:M, :ldc].float().cpu().to(torch.float64).numpy()


def _oracle(A, B, sa, sb, K, fa, fb, mode, block_m):
    return ofp8.gemm(A, B, K=K, fmt_a=fa, fmt_b=fb, mode=mode, scale_a=sa, scale_b=sb,
                     block_m=block_m)


SCALINGS = [("tensor", 1), ("block", 1), ("block", 128)]
PAIRS = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]


@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("mode,block_m", SCALINGS)
@pytest.mark.parametrize("out_dt", ["bf16", "fp16", "fp32"])
def test_fp8_every_element(fa, fb, mode, block_m, out_dt):
    # 300 x 280: a whole 256 tile and a ragged edge; K = 400 = 3 scale blocks
    # and a 16-deep tail; leading dimensions padded (NaN codes)
    M, N, K = 300, 280, 400
    say("case fp8 %s x %s %s/%d out=%s" % (fa, fb, mode, block_m, out_dt))
    A, B, sa, sb = make_fp8_operands(M, N, K, fa, fb, "uniform", seed=5, mode=mode,
                                     block_m=block_m, lda=K + 16, ldb=K + 32)
    h = new_handle()
    C = _run(h, A, B, sa, sb, K, fa, fb, mode, block_m, out_dt)
    h.close()
    Cr, S = _oracle(A, B, sa, sb, K, fa, fb, mode, block_m)
    err, worst = check(C, Cr, S, out_dt, "fp8 %s%s %s" % (fa, fb, mode))
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))


@pytest.mark.parametrize("mode,block_m", SCALINGS)
@pytest.mark.parametrize("splits", [None, 3])
def test_fp8_small_integers_bitwise(mode, block_m, splits):
    M, N, K = 300, 264, 512
    say("case fp8 int3 %s/%d splits=%s" % (mode, block_m, splits))
    A, B, sa, sb = make_fp8_operands(M, N, K, "e4m3", "e5m2", "int3", seed=7, mode=mode,
                                     block_m=block_m)
    h = new_handle("256x256x64_w8_pp2", splits)
    C = _run(h, A, B, sa, sb, K, "e4m3", "e5m2", mode, block_m, "fp32")
    h.close()
    Cr, _ = _oracle(A, B, sa, sb, K, "e4m3", "e5m2", mode, block_m)
    assert np.array_equal(C, Cr)


@pytest.mark.parametrize("mode,block_m", [("tensor", 1), ("block", 128)])
@pytest.mark.parametrize("out_dt,pad", [("fp32", 1), ("bf16", 3)])
def test_fp8_unaligned_ldc(mode, block_m, out_dt, pad):
    # rows of C not a multiple of 16 bytes apart: the stores take the
    # unaligned path; a whole 256 tile and ragged edges, padding left alone
    M, N, K = 300, 280, 256
    say("case fp8 ldc=N+%d %s %s/%d" % (pad, out_dt, mode, block_m))
    A, B, sa, sb = make_fp8_operands(M, N, K, "e4m3", "e4m3", "uniform", seed=9, mode=mode,
                                     block_m=block_m)
    h = new_handle()
    C = _run(h, A, B, sa, sb, K, "e4m3", "e4m3", mode, block_m, out_dt, ldc=N + pad)
    h.close()
    assert np.isnan(C[:, N:]).all()
    Cr, S = _oracle(A, B, sa, sb, K, "e4m3", "e4m3", mode, block_m)
    check(C[:, :N], Cr, S, out_dt, "fp8 ldc=N+%d" % pad)


@pytest.mark.parametrize("K", [16, 128, 144])
def test_fp8_short_k_bitwise(K):
    M, N = 260, 300
    for mode, block_m in SCALINGS:
        say("case fp8 short K=%d %s/%d" % (K, mode, block_m))
        A, B, sa, sb = make_fp8_operands(M, N, K, "e4m3", "e4m3", "int3", seed=K, mode=mode,
                                         block_m=block_m)
        h = new_handle()
        C = _run(h, A, B, sa, sb, K, "e4m3", "e4m3", mode, block_m, "fp32")
        h.close()
        Cr, _ = _oracle(A, B, sa, sb, K, "e4m3", "e4m3", mode, block_m)
        assert np.array_equal(C, Cr)


@pytest.mark.parametrize("block_m", [1, 128])
def test_fp8_zero_scales(block_m):
    # zero scales for some (row, k) blocks of A and some (column, k) blocks of
    # B: those blocks add nothing, the others keep their scale
    M, N, K = 300, 300, 640
    say("case fp8 zero scales block_m=%d" % block_m)
    A, B, sa, sb = make_fp8_operands(M, N, K, "e4m3", "e4m3", "int3", seed=3, mode="block",
                                     block_m=block_m)
    sa = sa.clone()
    sb = sb.clone()
    sa[::2, 1] = 0.0
    sa[:, 0] = 0.0                 # the first block of every row
    sb[1, 3] = 0.0
    sb[:, 4] = 0.0                 # the last block of every column
    h = new_handle()
    C = _run(h, A, B, sa, sb, K, "e4m3", "e4m3", "block", block_m, "fp32")
    h.close()
    Cr, _ = _oracle(A, B, sa, sb, K, "e4m3", "e4m3", "block", block_m)
    assert np.array_equal(C, Cr)


@pytest.mark.parametrize("mode,block_m", SCALINGS)
def test_fp8_decode_shape(mode, block_m):
    # M = 256 decode with split-K: the partials are summed by the second pass
    M, N, K = 256, 1024, 8192
    say("case fp8 decode %s/%d" % (mode, block_m))
    A, B, sa, sb = make_fp8_operands(M, N, K, "e4m3", "e4m3", "llm", seed=2, mode=mode,
                                     block_m=block_m)
    h = new_handle()
    C = _run(h, A, B, sa, sb, K, "e4m3", "e4m3", mode, block_m, "bf16")
    h.close()
    Cr, S = _oracle(A, B, sa, sb, K, "e4m3", "e4m3", mode, block_m)
    check(C, Cr, S, "bf16", "fp8 decode %s" % mode)


@pytest.mark.parametrize("mode,block_m", SCALINGS)
@pytest.mark.parametrize("splits", [None, 2])
def test_fp8_with_epilogue(mode, block_m, splits):
    M, N, K = 512, 300, 384
    say("case fp8 epilogue %s/%d splits=%s" % (mode, block_m, splits))
    A, B, sa, sb = make_fp8_operands(M, N, K, "e4m3", "e4m3", "uniform", seed=8, mode=mode,
                                     block_m=block_m)
    g = torch.Generator().manual_seed(8)
    C_old = (torch.rand((M, N), generator=g) * 4 - 2).to(torch.bfloat16)
    bias = (torch.rand(M, generator=g) * 2 - 1).to(torch.float32)
    bd = bias.to(DEV)
    epi = _lib.epilogue(0.5, -1.0, bd.data_ptr(), "m", "gelu")
    h = new_handle("256x256x64_w8_pp2", splits)
    D = _run(h, A, B, sa, sb, K, "e4m3", "e4m3", mode, block_m, "bf16", epi=epi, C_old=C_old)
    h.close()
    Cr, S = _oracle(A, B, sa, sb, K, "e4m3", "e4m3", mode, block_m)
    old = C_old.to(torch.float64).numpy()
    Dr = oepi.apply(Cr, C_old=old, alpha=0.5, beta=-1.0, bias=bias.numpy(), bias_along="m",
                    act="gelu")
    aS, t = oepi.scale_of(S, C_old=old, alpha=0.5, beta=-1.0, bias=bias.numpy(), bias_along="m")
    check_epilogue(D, Dr, aS, t, "bf16", "fp8 epilogue %s" % mode)


@pytest.mark.parametrize("mode,block_m", [("block", 1), ("tensor", 1)])
def test_fp8_full_size_sampled(mode, block_m):
    M = N = K = 4096
    say("case fp8 4096^3 %s sampled" % mode)
    A, B, sa, sb = make_fp8_operands(M, N, K, "e4m3", "e4m3", "uniform", seed=0, mode=mode,
                                     block_m=block_m)
    h = new_handle()
    C = _run(h, A, B, sa, sb, K, "e4m3", "e4m3", mode, block_m, "bf16")
    h.close()
    rng = np.random.default_rng(3)
    ii = np.concatenate([rng.integers(0, M, 3000), [0, M - 1, 0, M - 1]])
    jj = np.concatenate([rng.integers(0, N, 3000), [0, N - 1, N - 1, 0]])
    Cp, Sp = ofp8.gemm_points(A, B, ii, jj, K=K, mode=mode, scale_a=sa, scale_b=sb,
                              block_m=block_m)
    check(C[ii, jj], Cp, Sp, "bf16", "fp8 4096^3 %s points" % mode)


def test_fp8_torch_binding():
    from dense_gemm_nt_amd import gemm_fp8
    M, N, K = 272, 300, 256
    say("case fp8 torch binding")
    A, B, sa, sb = make_fp8_operands(M, N, K, "e4m3", "e5m2", "uniform", seed=1, mode="block",
                                     block_m=128)
    Ad = A.to(DEV).view(torch.float8_e4m3fn)
    Bd = B.to(DEV).view(torch.float8_e5m2)
    C = gemm_fp8(Ad, Bd, sa.to(DEV), sb.to(DEV), fmt_a="e4m3", fmt_b="e5m2",
                 out_dtype=torch.float32)
    Cr, S = _oracle(A, B, sa, sb, K, "e4m3", "e5m2", "block", 128)
    check(C.cpu().double().numpy(), Cr, S, "fp32", "fp8 binding")


def test_fp8_argument_checks():
    h = new_handle()
    X = torch.zeros((64, 64), dtype=torch.uint8, device=DEV)
    C = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    sc = torch.ones((64, 1), dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream(DEV).cuda_stream
    p = X.data_ptr()

    def st(M=16, N=16, K=32, lda=32, ldb=32, fa=3, fb=3, mode="tensor", block_m=1, sa=None,
           sb=None, hh=None):
        scales = _lib.fp8_scales(mode, sc.data_ptr() if sa is None else sa,
                                 sc.data_ptr() if sb is None else sb, block_m)
        return _lib.gemm_run_fp8((hh or h)._h, fa, fb, p, p, C.data_ptr(), M, N, K, lda, ldb, 64,
                                 0, scales, None, s)
    assert st() == _lib.GEMM_OK
    assert st(K=24, lda=32) == _lib.GEMM_ERR_UNSUPPORTED          # K % 16
    assert st(lda=40) == _lib.GEMM_ERR_MISALIGNED                 # lda % 16
    assert st(fa=0) == _lib.GEMM_ERR_UNSUPPORTED                  # not an FP8 format
    assert st(mode="block", block_m=64) == _lib.GEMM_ERR_INVALID_ARG
    assert st(sa=0) == _lib.GEMM_ERR_INVALID_ARG                  # null scale pointer
    assert st(sb=sc.data_ptr() + 2) == _lib.GEMM_ERR_INVALID_ARG  # misaligned scales
    assert _lib.gemm_run_fp8(h._h, 3, 3, p, p, C.data_ptr(), 16, 16, 32, 32, 32, 64, 0, None,
                             None, s) == _lib.GEMM_ERR_INVALID_ARG
    h2 = new_handle("128x128x64_w8_s4")
    assert st(hh=h2) == _lib.GEMM_ERR_UNSUPPORTED                 # only the pp2 tile
    torch.cuda.synchronize()
    h2.close()
    h.close()
