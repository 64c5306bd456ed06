"""Parity of the other operand layouts (gemm_run_layout, through the C ABI) with
the oracle: A and/or B stored MN-major (the transpose of the NT form's K-major
arrays), every element against oracle.gemm on the same stored arrays.

Cases: ragged M, N and a K tail with padded leading dimensions for both input
formats and two output formats; small-integer inputs (exact in FP32, so the
comparison is bitwise) with and without split-K and at short K; the skinny and
decode shapes; the fused epilogue; the 4096^3 and 1024 x 4096 x 4096 workloads
on sampled outputs; the torch binding's stride inference; and the argument
checks.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import epilogue as oepi
from dense_gemm_nt_amd import _lib
from gemm_inputs import make_operands, make_stored
from tests.gpu_util import CODE, TORCH_DT, new_handle, say
from tests.tolerance import check, check_epilogue

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
LAYOUT = {"k": _lib.GEMM_K_MAJOR, "mn": _lib.GEMM_MN_MAJOR}
OTHER = [("k", "mn"), ("mn", "k"), ("mn", "mn")]


def _run(h, la, lb, Xa, Xb, M, N, K, in_dt, out_dt, epi=None, C_old=None, ldc=None):
    """C on the GPU from stored arrays; C_old (host, out_dt) is C's prior content.
    Returns the stored rows of C, ldc (default N) columns wide."""
    lda, ldb = Xa.shape[1], Xb.shape[1]
    ldc = N if ldc is None else ldc
    Ad, Bd = Xa.to(DEV), Xb.to(DEV)
    if C_old is None:
        Cd = torch.full((max(M, 1), max(ldc, 1)), float("nan"), dtype=TORCH_DT[out_dt], device=DEV)
    else:
        Cd = C_old.to(DEV).clone()
    s = torch.cuda.current_stream(DEV)
    h.run_raw_layout(LAYOUT[la], LAYOUT[lb], Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), M, N, K,
                     lda, ldb, ldc, CODE[in_dt], CODE[out_dt], epi, s.cuda_stream)
    s.synchronize()
    return Cd[:M, :ldc].float().cpu().to(torch.float64).numpy()


def _views(Xa, Xb, la, lb, M, N, K):
    """The stored arrays cut to their logical extents (padding excluded)."""
    Va = Xa[:, :K] if la == "k" else Xa[:K, :M]
    Vb = Xb[:, :K] if lb == "k" else Xb[:K, :N]
    return Va, Vb


def _stored(M, N, K, la, lb, dt, dist, seed, pad=0):
    """make_stored with each leading dimension its row length rounded up to a
    multiple of 8 (the 16-byte row alignment the kernels need), plus `pad`."""
    def ld(layout, rows):
        ext = K if layout == "k" else rows
        return (ext + 7) // 8 * 8 + pad
    return make_stored(M, N, K, la, lb, dt, dist, seed=seed, lda=ld(la, M), ldb=ld(lb, N))


@pytest.mark.parametrize("la,lb", OTHER)
@pytest.mark.parametrize("in_dt", ["bf16", "fp16"])
@pytest.mark.parametrize("out_dt", ["bf16", "fp16", "fp32"])
def test_layout_every_element(la, lb, in_dt, out_dt):
    # 300 x 280: a whole 256 tile and a ragged edge both ways; K = 200 = 3 slabs
    # of 64 and a tail of 8; leading dimensions padded by 8 (NaN padding)
    M, N, K = 300, 280, 200
    say("case layout %s%s in=%s out=%s M=%d N=%d K=%d" % (la, lb, in_dt, out_dt, M, N, K))
    Xa, Xb = _stored(M, N, K, la, lb, in_dt, "uniform", seed=3, pad=8)
    h = new_handle()
    C = _run(h, la, lb, Xa, Xb, M, N, K, in_dt, out_dt)
    h.close()
    Va, Vb = _views(Xa, Xb, la, lb, M, N, K)
    Cr, S = oracle.gemm(Va, Vb, la, lb, in_dtype=in_dt)
    err, worst = check(C, Cr, S, out_dt, "layout %s%s" % (la, lb))
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))


@pytest.mark.parametrize("la,lb", OTHER)
@pytest.mark.parametrize("out_dt,pad", [("fp32", 1), ("bf16", 3)])
def test_layout_unaligned_ldc(la, lb, out_dt, pad):
    # rows of C not a multiple of 16 bytes apart on the MN-major kernels: the
    # unaligned store path, padding columns left alone
    M, N, K = 300, 280, 200
    say("case layout %s%s ldc=N+%d out=%s" % (la, lb, pad, out_dt))
    Xa, Xb = _stored(M, N, K, la, lb, "bf16", "uniform", seed=4)
    h = new_handle()
    C = _run(h, la, lb, Xa, Xb, M, N, K, "bf16", out_dt, ldc=N + pad)
    h.close()
    assert np.isnan(C[:, N:]).all()
    Va, Vb = _views(Xa, Xb, la, lb, M, N, K)
    Cr, S = oracle.gemm(Va, Vb, la, lb, in_dtype="bf16")
    check(C[:, :N], Cr, S, out_dt, "layout %s%s ldc=N+%d" % (la, lb, pad))


@pytest.mark.parametrize("la,lb", [("k", "k")] + OTHER)
@pytest.mark.parametrize("splits", [None, 2])
def test_layout_rotated_slab_order(la, lb, splits):
    # GEMM_ROTATE=2 on every layout: K-major operands run on the 128x128 tile
    # in the rotated k-slab order (K = 1000 is 15 slabs of 64 and a partial
    # last one, which keeps its place; 600 columns are three 256-column blocks,
    # so three different starts), MN-major ones on the ping-pong tile, in order.
    # Random values against the oracle, and small integers bitwise against the
    # natural order (exact sums, so any order gives the same bits).
    M, N, K = 100, 600, 1000
    say("case layout rotated order %s%s splits=%s" % (la, lb, splits))
    for dist in ("uniform", "int3"):
        Xa, Xb = _stored(M, N, K, la, lb, "bf16", dist, seed=6, pad=8)
        h2 = new_handle(None, splits, rotate=2)
        C = _run(h2, la, lb, Xa, Xb, M, N, K, "bf16", "fp32")
        h2.close()
        Va, Vb = _views(Xa, Xb, la, lb, M, N, K)
        Cr, S = oracle.gemm(Va, Vb, la, lb, in_dtype="bf16")
        if dist == "uniform":
            check(C, Cr, S, "fp32", "layout %s%s rotated" % (la, lb))
        else:
            h0 = new_handle(None, splits, rotate=0)
            C0 = _run(h0, la, lb, Xa, Xb, M, N, K, "bf16", "fp32")
            h0.close()
            assert np.array_equal(C, Cr) and np.array_equal(C0, Cr)


@pytest.mark.parametrize("la,lb", OTHER)
@pytest.mark.parametrize("splits", [None, 3])
def test_layout_small_integers_bitwise(la, lb, splits):
    M, N, K = 512, 300, 1000
    say("case layout int3 %s%s splits=%s" % (la, lb, splits))
    Xa, Xb = _stored(M, N, K, la, lb, "bf16", "int3", seed=8)
    h = new_handle("256x256x64_w8_pp2", splits)
    C = _run(h, la, lb, Xa, Xb, M, N, K, "bf16", "fp32")
    h.close()
    Cr, _ = oracle.gemm(*_views(Xa, Xb, la, lb, M, N, K), la, lb, in_dtype="bf16")
    assert np.array_equal(C, Cr)


@pytest.mark.parametrize("la,lb", OTHER)
@pytest.mark.parametrize("K", [8, 64, 72, 128])
def test_layout_short_k_bitwise(la, lb, K):
    M, N = 300, 280
    say("case layout short K %s%s K=%d" % (la, lb, K))
    Xa, Xb = _stored(M, N, K, la, lb, "fp16", "int3", seed=K)
    h = new_handle()
    C = _run(h, la, lb, Xa, Xb, M, N, K, "fp16", "fp32")
    h.close()
    Cr, _ = oracle.gemm(*_views(Xa, Xb, la, lb, M, N, K), la, lb, in_dtype="fp16")
    assert np.array_equal(C, Cr)


@pytest.mark.parametrize("M,N", [(301, 279), (1, 333), (333, 1), (7, 9)])
def test_layout_odd_extents_bitwise(M, N):
    # an odd row length puts the last element of a stored row in the first
    # half of a 4-byte word: it must still be read
    K = 136
    for la, lb in OTHER:
        say("case layout odd extents %s%s M=%d N=%d" % (la, lb, M, N))
        Xa, Xb = _stored(M, N, K, la, lb, "bf16", "int3", seed=M + N)
        h = new_handle()
        C = _run(h, la, lb, Xa, Xb, M, N, K, "bf16", "fp32")
        h.close()
        Cr, _ = oracle.gemm(*_views(Xa, Xb, la, lb, M, N, K), la, lb, in_dtype="bf16")
        assert np.array_equal(C, Cr), (la, lb)


@pytest.mark.parametrize("la,lb", [("k", "k")] + OTHER)
def test_layouts_agree_with_nt_bitwise(la, lb):
    # the same logical operands in any layout feed the same MFMA sequence
    M, N, K = 512, 512, 512
    say("case layout vs NT %s%s" % (la, lb))
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=4)
    h = new_handle()
    Cnt = _run(h, "k", "k", A, B, M, N, K, "bf16", "fp32")
    Xa, Xb = make_stored(M, N, K, la, lb, "bf16", "uniform", seed=4)
    C = _run(h, la, lb, Xa, Xb, M, N, K, "bf16", "fp32")
    h.close()
    assert np.array_equal(C, Cnt)


@pytest.mark.parametrize("M,N,K", [(1, 1000, 4096), (16, 520, 2048), (256, 512, 4096),
                                   (130, 8, 64)])
def test_layout_decode_shapes(M, N, K):
    # small M: one 256-row tile, split-K over the compute units
    for la, lb in OTHER:
        say("case layout decode %s%s M=%d N=%d K=%d" % (la, lb, M, N, K))
        Xa, Xb = _stored(M, N, K, la, lb, "bf16", "llm", seed=M)
        h = new_handle()
        C = _run(h, la, lb, Xa, Xb, M, N, K, "bf16", "bf16")
        h.close()
        Cr, S = oracle.gemm(*_views(Xa, Xb, la, lb, M, N, K), la, lb, in_dtype="bf16")
        check(C, Cr, S, "bf16", "layout decode %s%s" % (la, lb))


@pytest.mark.parametrize("la,lb", OTHER)
@pytest.mark.parametrize("splits", [None, 2])
def test_layout_with_epilogue(la, lb, splits):
    M, N, K = 512, 300, 320
    say("case layout epilogue %s%s splits=%s" % (la, lb, splits))
    Xa, Xb = _stored(M, N, K, la, lb, "bf16", "uniform", seed=6)
    g = torch.Generator().manual_seed(6)
    C_old = (torch.rand((M, N), generator=g) * 4 - 2).to(torch.bfloat16)
    bias = (torch.rand(N, generator=g) * 2 - 1).to(torch.float32)
    bd = bias.to(DEV)
    epi = _lib.epilogue(-0.75, 0.5, bd.data_ptr(), "n", "gelu")
    h = new_handle("256x256x64_w8_pp2", splits)
    D = _run(h, la, lb, Xa, Xb, M, N, K, "bf16", "bf16", epi=epi, C_old=C_old)
    h.close()
    Cr, S = oracle.gemm(*_views(Xa, Xb, la, lb, M, N, K), la, lb, in_dtype="bf16")
    old = C_old.to(torch.float64).numpy()
    Dr = oepi.apply(Cr, C_old=old, alpha=-0.75, beta=0.5, bias=bias.numpy(), bias_along="n",
                    act="gelu")
    aS, t = oepi.scale_of(S, C_old=old, alpha=-0.75, beta=0.5, bias=bias.numpy(), bias_along="n")
    check_epilogue(D, Dr, aS, t, "bf16", "layout epilogue %s%s" % (la, lb))


@pytest.mark.parametrize("M,N,K,la,lb", [(4096, 4096, 4096, "k", "mn"),
                                         (1024, 4096, 4096, "k", "mn"),
                                         (4096, 4096, 4096, "mn", "mn")])
def test_layout_full_size_sampled(M, N, K, la, lb):
    # row-major A times row-major B (the NN form), at the square and skinny sizes
    say("case layout full size %s%s M=%d N=%d K=%d" % (la, lb, M, N, K))
    Xa, Xb = make_stored(M, N, K, la, lb, "bf16", "uniform", seed=1)
    h = new_handle()
    C = _run(h, la, lb, Xa, Xb, M, N, K, "bf16", "bf16")
    h.close()
    rng = np.random.default_rng(2)
    ii = np.concatenate([rng.integers(0, M, 3000), [0, M - 1, 0, M - 1]])
    jj = np.concatenate([rng.integers(0, N, 3000), [0, N - 1, N - 1, 0]])
    Cp, Sp = oracle.gemm_points(Xa, Xb, ii, jj, la, lb, in_dtype="bf16")
    check(C[ii, jj], Cp, Sp, "bf16", "layout %s%s %dx%dx%d points" % (la, lb, M, N, K))


def test_torch_binding_infers_layouts_from_strides():
    from dense_gemm_nt_amd import gemm_nt
    M, N, K = 304, 264, 136
    say("case torch binding layouts")
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=12)
    Ad, Bd = A.to(DEV), B.to(DEV)
    W = Bd.t().contiguous()        # [K, N] row-major: B = W.t() is N-major
    At = Ad.t().contiguous()       # [K, M] row-major: A = At.t() is M-major
    Cr, S = oracle.gemm_nt(A, B, in_dtype="bf16")
    for a, b in ((Ad, W.t()), (At.t(), Bd), (At.t(), W.t()), (Ad, Bd)):
        C = gemm_nt(a, b, out_dtype=torch.float32)
        check(C.cpu().double().numpy(), Cr, S, "fp32", "binding")
    with pytest.raises(ValueError):
        gemm_nt(Ad[:, ::2], Bd[:, ::2])           # neither stride is 1


def test_layout_argument_checks():
    h = new_handle()
    X = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    C = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.current_stream(DEV).cuda_stream
    p = X.data_ptr()

    def st(la, lb, M, N, K, lda, ldb, hh=None):
        return _lib.gemm_run_layout((hh or h)._h, la, lb, p, p, C.data_ptr(), M, N, K, lda, ldb,
                                    64, 0, 0, None, s)
    assert st(1, 0, 16, 16, 12, 16, 16) == _lib.GEMM_ERR_UNSUPPORTED    # K % 8 with MN-major
    assert st(1, 0, 32, 16, 16, 16, 16) == _lib.GEMM_ERR_INVALID_ARG    # lda < M
    assert st(0, 1, 16, 32, 16, 16, 16) == _lib.GEMM_ERR_INVALID_ARG    # ldb < N
    assert st(1, 0, 16, 16, 16, 20, 16) == _lib.GEMM_ERR_MISALIGNED     # lda % 8
    assert st(2, 0, 16, 16, 16, 16, 16) == _lib.GEMM_ERR_INVALID_ARG    # no such layout
    assert st(0, 0, 16, 16, 12, 16, 16) == _lib.GEMM_OK                 # NT takes any K
    assert st(1, 1, 16, 16, 16, 16, 16) == _lib.GEMM_OK
    h2 = new_handle("128x128x64_w8_s4")
    assert st(1, 1, 16, 16, 16, 16, 16, hh=h2) == _lib.GEMM_ERR_UNSUPPORTED  # only the pp2 tile
    torch.cuda.synchronize()
    h2.close()
    h.close()
