"""Parity of the fused epilogue (gemm_run_ex, through the C ABI) with the oracle.

D = act(alpha * A.B^T + beta * C_old + bias) is compared element by element with
oracle.epilogue.apply on the exact product, within tests/tolerance.check_epilogue;
with small-integer inputs and exactly representable scalars every FP32 step is
exact, so there the comparison is bitwise.  Every kernel family member that has
its own store path is forced once: the staged whole-tile store (256x256 tiles),
the direct store (edge tiles, 128x128), and the split-K sum.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import epilogue as oepi
from dense_gemm_nt_amd import _lib
from gemm_inputs import make_operands
from tests.gpu_util import CODE, TORCH_DT, new_handle, say
from tests.tolerance import check_epilogue

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def _run_ex(h, A, B, K, in_dt, out_dt, C_old, alpha, beta, bias, along, act):
    """D on the GPU; C_old (host tensor in out_dt) is the prior content of C."""
    M, lda = A.shape
    N, ldb = B.shape
    Ad, Bd = A.to(DEV), B.to(DEV)
    Cd = C_old.to(DEV).clone()
    bd = bias.to(DEV) if bias is not None else None
    epi = _lib.epilogue(alpha, beta, bd.data_ptr() if bd is not None else 0, along, act)
    s = torch.cuda.current_stream(DEV)
    h.run_raw_ex(Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), M, N, K, lda, ldb, N,
                 CODE[in_dt], CODE[out_dt], epi, s.cuda_stream)
    s.synchronize()
    return Cd.float().cpu().to(torch.float64).numpy()


def _case(M, N, K, in_dt, out_dt, alpha, beta, along, act, seed, config=None, splits=None,
          dist="uniform"):
    A, B = make_operands(M, N, K, in_dt, dist, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    C_old = (torch.rand((M, N), generator=g) * 4 - 2).to(TORCH_DT[out_dt])
    bias = None
    if along != "none":
        nb = N if along == "n" else M
        bias = (torch.rand(nb, generator=g) * 2 - 1).to(torch.float32)
    h = new_handle(config, splits)
    D = _run_ex(h, A, B, K, in_dt, out_dt, C_old, alpha, beta, bias, along, act)
    h.close()
    Cr, S = oracle.gemm_nt(A, B, K=K, in_dtype=in_dt)
    old = C_old.to(torch.float64).numpy()
    b = bias.numpy() if bias is not None else None
    Dr = oepi.apply(Cr, C_old=old, alpha=alpha, beta=beta, bias=b, bias_along=along, act=act)
    aS, t = oepi.scale_of(S, C_old=old, alpha=alpha, beta=beta, bias=b, bias_along=along)
    return check_epilogue(D, Dr, aS, t, out_dt, "M=%d N=%d K=%d %s" % (M, N, K, act))


EPIS = [
    # alpha, beta, bias along, activation
    (0.5, 0.0, "n", "relu"),
    (-1.25, 0.75, "m", "gelu"),
    (1.0, 1.0, "none", "none"),
    (2.0, -0.5, "n", "none"),
    (1.0, 0.0, "none", "gelu"),
]


@pytest.mark.parametrize("config,splits", [("256x256x64_w8_pp2", None), ("128x128x64_w8_s4", None),
                                           ("256x256x64_w8_pp2", 3), ("32x128x64_w4_s6", None),
                                           ("32x128x64_w4_s6", 3), ("128x128x64_w8_s4", 2)])
@pytest.mark.parametrize("alpha,beta,along,act", EPIS)
@pytest.mark.parametrize("out_dt", ["bf16", "fp32"])
def test_epilogue_every_element(config, splits, alpha, beta, along, act, out_dt):
    # 512 x 300: two whole 256-row tiles and a ragged column edge
    say("case epilogue %s splits=%s a=%g b=%g bias=%s act=%s out=%s" % (config, splits, alpha, beta,
                                                                       along, act, out_dt))
    err, worst = _case(512, 300, 328, "bf16", out_dt, alpha, beta, along, act, seed=7,
                       config=config, splits=splits)
    say("  max|err|=%.3g worst/bound=%.3g" % (err, worst))


@pytest.mark.parametrize("M,N,K", [(256, 8192, 1024), (130, 257, 64), (1, 300, 40)])
def test_epilogue_default_plans_fp16(M, N, K):
    say("case epilogue default plan fp16 M=%d N=%d K=%d" % (M, N, K))
    _case(M, N, K, "fp16", "fp16", 0.75, 0.5, "n", "gelu", seed=M + N)


def test_epilogue_small_integers_bitwise():
    # int3 inputs, alpha = 2, beta = 1, integer C_old and bias, ReLU: all exact in FP32
    M, N, K = 300, 280, 1000
    say("case epilogue int3 bitwise")
    A, B = make_operands(M, N, K, "bf16", "int3", seed=21)
    g = torch.Generator().manual_seed(3)
    C_old = torch.randint(-50, 50, (M, N), generator=g).to(torch.float32)
    bias = torch.randint(-20, 20, (N,), generator=g).to(torch.float32)
    for config in ("256x256x64_w8_pp2", "128x128x64_w8_s4"):
        h = new_handle(config)
        D = _run_ex(h, A, B, K, "bf16", "fp32", C_old, 2.0, 1.0, bias, "n", "relu")
        h.close()
        Cr, _ = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
        Dr = oepi.apply(Cr, C_old=C_old.numpy().astype(np.float64), alpha=2.0, beta=1.0,
                        bias=bias.numpy(), bias_along="n", act="relu")
        assert np.array_equal(D, Dr), config


def test_epilogue_full_size_sampled():
    # the 4096^3 workload with a bias and GELU, compared on sampled points
    M = N = K = 4096
    say("case epilogue 4096^3 bias+gelu sampled")
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=0)
    g = torch.Generator().manual_seed(9)
    bias = (torch.rand(N, generator=g) * 2 - 1).to(torch.float32)
    Ad, Bd, bd = A.to(DEV), B.to(DEV), bias.to(DEV)
    from dense_gemm_nt_amd import gemm_nt
    D = gemm_nt(Ad, Bd, bias=bd, bias_along="n", activation="gelu").float().cpu().double().numpy()
    rng = np.random.default_rng(4)
    ii, jj = rng.integers(0, M, 3000), rng.integers(0, N, 3000)
    Cp, Sp = oracle.gemm_nt_points(A, B, ii, jj, K=K, in_dtype="bf16")
    b = bias.numpy()
    # the sampled points as one 1 x P output row whose column p has bias b[jj[p]]
    Dr = oepi.apply(Cp[None, :], bias=b[jj], bias_along="n", act="gelu")[0]
    aS = Sp
    t = np.abs(b[jj].astype(np.float64))
    check_epilogue(D[ii, jj], Dr, aS, t, "bf16", "4096^3 gelu points")


def test_epilogue_rejects_bad_descriptors():
    h = new_handle()
    A = torch.zeros((4, 8), dtype=torch.bfloat16, device=DEV)
    C = torch.zeros((4, 4), dtype=torch.bfloat16, device=DEV)
    bias = torch.zeros(8, dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream(DEV).cuda_stream

    def st(epi):
        return _lib.gemm_run_ex(h._h, A.data_ptr(), A.data_ptr(), C.data_ptr(), 4, 4, 8, 8, 8, 4,
                                0, 0, epi, s)
    assert st(_lib.GemmEpilogue(1.0, 0.0, None, 1, 0)) == _lib.GEMM_ERR_INVALID_ARG      # no bias
    assert st(_lib.GemmEpilogue(1.0, 0.0, bias.data_ptr() + 2, 1, 0)) == _lib.GEMM_ERR_INVALID_ARG
    assert st(_lib.GemmEpilogue(1.0, 0.0, None, 0, 7)) == _lib.GEMM_ERR_INVALID_ARG      # activation
    assert st(_lib.GemmEpilogue(1.0, 0.0, None, 5, 0)) == _lib.GEMM_ERR_INVALID_ARG      # bias axis
    assert st(_lib.GemmEpilogue(float("inf"), 0.0, None, 0, 0)) == _lib.GEMM_ERR_UNSUPPORTED
    assert st(None) == _lib.GEMM_OK
    torch.cuda.synchronize()
    h.close()
