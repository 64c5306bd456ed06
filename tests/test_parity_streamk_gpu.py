"""Parity of the stream-K decomposition with the CPU oracle, through the C ABI.

Stream-K (CuTe page, section 9, named beside split-K) gives every workgroup an
equal run of the tiles * k-slabs units of the 256x256 ping-pong tile; each tile
a run touches yields one FP32 partial, and a second kernel adds a tile's
partials in workgroup order.  The mode is forced here (GEMM_STREAMK=2 with the
ping-pong tile) on shapes whose runs cut tiles at arbitrary k-slabs, ragged
tiles included, so that many partials meet in one tile.  Small-integer inputs
make every partial sum exact: those comparisons are bitwise.  The fused epilogue
runs in the reduction kernel and is checked against oracle.epilogue.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import epilogue as oepi
from dense_gemm_nt_amd import _lib, gemm_plan
from gemm_inputs import make_operands
from tests.gpu_util import CODE, TORCH_DT, compare_full, new_handle, run_gpu, say
from tests.tolerance import check, check_epilogue

pytestmark = pytest.mark.gpu

PP2 = "256x256x64_w8_pp2"
DEV = torch.device("cuda", 0)


def ld8(x):
    return (x + 7) // 8 * 8


def _bits(x):
    return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# M, N, K: runs of 1-2 k-slabs (many partials per tile), ragged edges
SHAPES = [(300, 280, 1000), (257, 513, 4104), (1000, 700, 2048), (64, 300, 640)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_streamk_small_integers_bitwise(M, N, K):
    say("case stream-K int3 M=%d N=%d K=%d" % (M, N, K))
    h = new_handle(PP2, streamk=2)
    A, B = make_operands(M, N, K, "bf16", "int3", seed=7, lda=ld8(K + 1), ldb=ld8(K + 3))
    C = run_gpu(h, A, B, K, "bf16", "fp32")
    Cr, _ = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    assert np.array_equal(C, Cr)
    Cb = run_gpu(h, A, B, K, "bf16", "bf16", keep_device=True)
    assert np.array_equal(_bits(Cb), oracle.encode(Cr, "bf16"))
    h.close()


@pytest.mark.parametrize("in_dt,out_dt", [("fp16", "fp32"), ("bf16", "bf16")])
def test_streamk_random_every_element(in_dt, out_dt):
    M, N, K = 1000, 700, 2048
    say("case stream-K random M=%d N=%d K=%d %s->%s" % (M, N, K, in_dt, out_dt))
    h = new_handle(PP2, streamk=2)
    A, B = make_operands(M, N, K, in_dt, "uniform", seed=11)
    C = run_gpu(h, A, B, K, in_dt, out_dt, ldc=N + 3)
    err, worst = compare_full(C, A, B, K, in_dt, out_dt, "stream-K M=%d N=%d K=%d" % (M, N, K))
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))
    # the partials are added in a fixed order: a second call gives the same bits
    C2 = run_gpu(h, A, B, K, in_dt, out_dt, ldc=N + 3)
    assert np.array_equal(C, C2)
    h.close()


@pytest.mark.parametrize("alpha,beta,along,act", [(-1.25, 0.75, "m", "gelu"), (0.5, 0.0, "n", "relu")])
def test_streamk_fused_epilogue(alpha, beta, along, act):
    M, N, K = 300, 280, 1000
    say("case stream-K epilogue alpha=%g beta=%g bias=%s act=%s" % (alpha, beta, along, act))
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=3)
    g = torch.Generator().manual_seed(4)
    C_old = (torch.rand((M, N), generator=g) * 4 - 2).to(TORCH_DT["bf16"])
    nb = N if along == "n" else M
    bias = (torch.rand(nb, generator=g) * 2 - 1).to(torch.float32)
    h = new_handle(PP2, streamk=2)
    Ad, Bd, Cd, bd = A.to(DEV), B.to(DEV), C_old.to(DEV).clone(), bias.to(DEV)
    epi = _lib.epilogue(alpha, beta, bd.data_ptr(), along, act)
    s = torch.cuda.current_stream(DEV)
    h.run_raw_ex(Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), M, N, K, K, K, N,
                 CODE["bf16"], CODE["bf16"], epi, s.cuda_stream)
    s.synchronize()
    D = Cd.float().cpu().to(torch.float64).numpy()
    h.close()
    Cr, S = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    old = C_old.to(torch.float64).numpy()
    Dr = oepi.apply(Cr, C_old=old, alpha=alpha, beta=beta, bias=bias.numpy(), bias_along=along, act=act)
    aS, t = oepi.scale_of(S, C_old=old, alpha=alpha, beta=beta, bias=bias.numpy(), bias_along=along)
    check_epilogue(D, Dr, aS, t, "bf16", "stream-K epilogue")


def test_streamk_is_planned_for_few_tiles_with_long_k(capfd):
    # (3000, 3000, 5000): 144 tiles, runs of ~44 k-slabs; the default plan runs
    # it as stream-K (the log line of the call says so), GEMM_STREAMK=0 as the
    # plain plan, and both agree with the oracle
    M, N, K = 3000, 3000, 5000
    p = gemm_plan(M, N, K, _lib.GEMM_FP16, _lib.GEMM_FP32)
    assert p["streamk"] == 1 and p["workgroups"] == 256
    A, B = make_operands(M, N, K, "fp16", "uniform", seed=5)
    Cr, S = oracle.gemm_nt(A, B, K=K, in_dtype="fp16")
    for streamk, tag in ((None, "stream-K"), (0, "")):
        say("case stream-K rule M=%d N=%d K=%d fp16->fp32 GEMM_STREAMK=%s" % (M, N, K, streamk))
        os.environ["GEMM_LOG"] = "1"
        try:
            h = new_handle(streamk=streamk)
        finally:
            os.environ.pop("GEMM_LOG", None)
        capfd.readouterr()
        C = run_gpu(h, A, B, K, "fp16", "fp32")
        err = capfd.readouterr().err
        h.close()
        if tag:
            assert tag in err and "grid=256" in err, err
        else:
            assert "stream-K" not in err and "grid=144" in err, err
        check(C, Cr, S, "fp32", "GEMM_STREAMK=%s" % streamk)
