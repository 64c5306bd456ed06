"""Parity of the grouped GEMM (gemm_run_grouped, through the C ABI) with the
oracle (oracle.gemm_grouped): every element of every group, on a problem list
with ragged, tiny, empty and K = 0 groups; bitwise on small integers; the fused
epilogue with a bias per group; a mixture-of-experts list at full size on
sampled outputs; bitwise agreement with one launch per group; argument checks.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import epilogue as oepi
from dense_gemm_nt_amd import _lib
from gemm_inputs import make_operands
from tests.gpu_util import CODE, TORCH_DT, new_handle, say
from tests.tolerance import check, check_epilogue

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)

# (M, N, K): ragged edges, a one-row group, empty groups, K = 0, a K tail
SHAPES = [(300, 280, 200), (1, 256, 64), (0, 100, 64), (513, 130, 136), (64, 700, 512),
          (256, 256, 0), (7, 0, 32), (129, 33, 8)]


def _problems(shapes, dt, dist, seed, out_dt, C_old=None, biases=None):
    host, dev, outs = [], [], []
    for g, (M, N, K) in enumerate(shapes):
        A, B = make_operands(M, N, K, dt, dist, seed=seed + g)
        host.append((A, B, K))
        Ad, Bd = A.to(DEV), B.to(DEV)
        if C_old is not None:
            Cd = C_old[g].to(DEV).clone()
        else:
            Cd = torch.full((M, N), float("nan"), dtype=TORCH_DT[out_dt], device=DEV)
        bd = biases[g].to(DEV) if biases is not None else None
        dev.append((Ad, Bd, Cd, bd))
        outs.append(Cd)
    probs = [_lib.GemmGroupProblem(Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(),
                                   bd.data_ptr() if bd is not None else None, M, N, K,
                                   max(K, 1), max(K, 1), max(N, 1))
             for (Ad, Bd, Cd, bd), (M, N, K) in zip(dev, shapes)]
    return host, dev, probs, outs


def _launch(h, probs, dt, out_dt, epi=None):
    s = torch.cuda.current_stream(DEV)
    st = _lib.gemm_run_grouped(h._h, probs, CODE[dt], CODE[out_dt], epi, s.cuda_stream)
    s.synchronize()
    return st


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("out_dt", ["bf16", "fp16", "fp32"])
def test_grouped_every_element(dt, out_dt):
    say("case grouped %s -> %s, %d groups" % (dt, out_dt, len(SHAPES)))
    host, dev, probs, outs = _problems(SHAPES, dt, "uniform", 11, out_dt)
    h = new_handle()
    assert _launch(h, probs, dt, out_dt) == _lib.GEMM_OK
    h.close()
    for g, ((Cr, S), C) in enumerate(zip(oracle.gemm_grouped(host, in_dtype=dt), outs)):
        check(C.float().cpu().double().numpy(), Cr, S, out_dt, "group %d %r" % (g, SHAPES[g]))


@pytest.mark.parametrize("out_dt", ["fp32", "bf16"])
def test_grouped_unaligned_ldc(out_dt):
    # each group's C rows a different, unaligned number of elements apart;
    # the padding columns stay untouched
    shapes = [(300, 280, 200), (64, 700, 512), (3, 129, 72)]
    pads = [1, 3, 5]
    say("case grouped ldc=N+pad %s" % out_dt)
    host, dev, outs = [], [], []
    for g, ((M, N, K), pad) in enumerate(zip(shapes, pads)):
        A, B = make_operands(M, N, K, "bf16", "uniform", seed=30 + g)
        host.append((A, B, K))
        Ad, Bd = A.to(DEV), B.to(DEV)
        Cd = torch.full((M, N + pad), float("nan"), dtype=TORCH_DT[out_dt], device=DEV)
        dev.append((Ad, Bd, Cd))
    probs = [_lib.GemmGroupProblem(Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), None, M, N, K, K, K,
                                   N + pad)
             for (Ad, Bd, Cd), (M, N, K), pad in zip(dev, shapes, pads)]
    h = new_handle()
    assert _launch(h, probs, "bf16", out_dt) == _lib.GEMM_OK
    h.close()
    for g, ((Cr, S), (_, _, Cd), (M, N, K)) in enumerate(zip(oracle.gemm_grouped(host), dev, shapes)):
        C = Cd.float().cpu().double().numpy()
        assert np.isnan(C[:, N:]).all(), g
        check(C[:, :N], Cr, S, out_dt, "group %d ldc=N+%d" % (g, pads[g]))


def test_grouped_small_integers_bitwise():
    say("case grouped int3 bitwise")
    host, dev, probs, outs = _problems(SHAPES, "bf16", "int3", 5, "fp32")
    h = new_handle()
    assert _launch(h, probs, "bf16", "fp32") == _lib.GEMM_OK
    h.close()
    for g, ((Cr, _), C) in enumerate(zip(oracle.gemm_grouped(host), outs)):
        assert np.array_equal(C.cpu().double().numpy(), Cr), g


@pytest.mark.parametrize("shapes", [
    [(300, 280, 2048), (512, 512, 1024), (40, 300, 512)],
    # a mixture-of-experts token mix, one tile row each: A loads wholly past a
    # problem's rows re-read its row 0 in the grouped launch and read zeros in
    # a plain one; the outputs they feed are never stored
    [(m, 512, 1024) for m in (64, 17, 200, 3, 90, 128, 256, 40, 1, 129)]])
def test_grouped_matches_one_launch_per_group_bitwise(shapes):
    # the same tile kernel without K splits: the same MFMA order, the same bits
    say("case grouped vs per-group launches, %d groups" % len(shapes))
    host, dev, probs, outs = _problems(shapes, "bf16", "uniform", 2, "bf16")
    h = new_handle()
    assert _launch(h, probs, "bf16", "bf16") == _lib.GEMM_OK
    h.close()
    h1 = new_handle("256x256x64_w8_pp2", 1)
    s = torch.cuda.current_stream(DEV)
    for (Ad, Bd, Cd, _), (M, N, K) in zip(dev, shapes):
        C1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        h1.run_raw(Ad.data_ptr(), Bd.data_ptr(), C1.data_ptr(), M, N, K, K, K, N, 0, 0,
                   s.cuda_stream)
        s.synchronize()
        assert torch.equal(C1.view(torch.int16), Cd.view(torch.int16))
    h1.close()


@pytest.mark.parametrize("along", ["n", "m"])
def test_grouped_with_epilogue(along):
    shapes = [s for s in SHAPES if s[0] and s[1]]
    say("case grouped epilogue bias along %s" % along)
    g = torch.Generator().manual_seed(4)
    C_old = [(torch.rand((M, N), generator=g) * 4 - 2).to(torch.bfloat16) for M, N, _ in shapes]
    biases = [(torch.rand(N if along == "n" else M, generator=g) * 2 - 1).to(torch.float32)
              for M, N, _ in shapes]
    host, dev, probs, outs = _problems(shapes, "bf16", "uniform", 9, "bf16", C_old, biases)
    epi = _lib.epilogue(1.5, 0.25, 0, along, "gelu")
    h = new_handle()
    assert _launch(h, probs, "bf16", "bf16", epi) == _lib.GEMM_OK
    h.close()
    for i, ((Cr, S), D) in enumerate(zip(oracle.gemm_grouped(host), outs)):
        old = C_old[i].to(torch.float64).numpy()
        b = biases[i].numpy()
        Dr = oepi.apply(Cr, C_old=old, alpha=1.5, beta=0.25, bias=b, bias_along=along, act="gelu")
        aS, t = oepi.scale_of(S, C_old=old, alpha=1.5, beta=0.25, bias=b, bias_along=along)
        check_epilogue(D.float().cpu().double().numpy(), Dr, aS, t, "bf16", "group %d" % i)


def test_grouped_moe_sampled():
    # eight experts of a mixture-of-experts layer: tokens per expert uneven,
    # each expert's weight [N, K]; compared on sampled outputs
    tokens = [1024, 3000, 512, 2048, 7, 2500, 4000, 1293]
    N, K = 2048, 4096
    shapes = [(m, N, K) for m in tokens]
    say("case grouped MoE 8 experts N=%d K=%d" % (N, K))
    host, dev, probs, outs = _problems(shapes, "bf16", "llm", 20, "bf16")
    h = new_handle()
    assert _launch(h, probs, "bf16", "bf16") == _lib.GEMM_OK
    h.close()
    rng = np.random.default_rng(1)
    for g, ((A, B, _), C) in enumerate(zip(host, outs)):
        M = A.shape[0]
        ii = np.concatenate([rng.integers(0, M, 400), [0, M - 1]])
        jj = np.concatenate([rng.integers(0, N, 400), [N - 1, 0]])
        Cp, Sp = oracle.gemm_nt_points(A, B, ii, jj, K=K)
        check(C.float().cpu().double().numpy()[ii, jj], Cp, Sp, "bf16", "expert %d" % g)


def test_grouped_argument_checks():
    h = new_handle()
    X = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(64, dtype=torch.float32, device=DEV)
    p = X.data_ptr()

    def prob(M=16, N=16, K=16, lda=16, bias=None):
        return _lib.GemmGroupProblem(p, p, p, bias, M, N, K, lda, 16, 16)

    s = torch.cuda.current_stream(DEV).cuda_stream
    run = lambda probs, epi=None: _lib.gemm_run_grouped(h._h, probs, 0, 0, epi, s)
    assert run([prob(), prob()]) == _lib.GEMM_OK
    assert run([]) == _lib.GEMM_OK
    assert run([prob(), prob(K=12, lda=16)]) == _lib.GEMM_ERR_UNSUPPORTED   # K % 8
    assert run([prob(lda=8)]) == _lib.GEMM_ERR_INVALID_ARG                 # lda < K
    assert run([prob()], _lib.epilogue(1.0, 0.0, b.data_ptr(), "n")) == _lib.GEMM_ERR_INVALID_ARG
    assert run([prob()], _lib.epilogue(1.0, 0.0, 0, "n")) == _lib.GEMM_ERR_INVALID_ARG  # no bias
    assert run([prob(bias=b.data_ptr())], _lib.epilogue(1.0, 0.0, 0, "n")) == _lib.GEMM_OK
    assert _lib.lib().gemm_run_grouped(h._h, None, 2, 0, 0, None, s) == _lib.GEMM_ERR_INVALID_ARG
    torch.cuda.synchronize()
    h.close()


def test_grouped_torch_binding():
    from dense_gemm_nt_amd import gemm_grouped
    shapes = [(100, 300, 64), (257, 64, 128)]
    say("case grouped torch binding")
    As, Bs, host = [], [], []
    for g, (M, N, K) in enumerate(shapes):
        A, B = make_operands(M, N, K, "fp16", "uniform", seed=g)
        host.append((A, B, K))
        As.append(A.to(DEV))
        Bs.append(B.to(DEV))
    Cs = gemm_grouped(As, Bs, out_dtype=torch.float32)
    for (Cr, S), C in zip(oracle.gemm_grouped(host, in_dtype="fp16"), Cs):
        check(C.cpu().double().numpy(), Cr, S, "fp32", "binding")


def test_grouped_back_to_back_calls_reuse_the_staging():
    # three grouped calls queued on one stream with no wait between them, each
    # with its own problem list: every call reads its own list
    h = new_handle()
    s = torch.cuda.current_stream(DEV)
    lists = [[(300, 280, 64), (17, 512, 128)], [(600, 40, 256)], [(1, 8, 8), (256, 256, 72), (90, 90, 16)]]
    runs = []
    for li, shapes in enumerate(lists):
        say("case grouped back-to-back list %d" % li)
        host, dev, probs, outs = _problems(shapes, "bf16", "int3", 40 + li, "fp32")
        st = _lib.gemm_run_grouped(h._h, probs, CODE["bf16"], CODE["fp32"], None, s.cuda_stream)
        assert st == _lib.GEMM_OK
        runs.append((host, dev, outs))
    s.synchronize()
    h.close()
    for host, _, outs in runs:
        for (Cr, _), C in zip(oracle.gemm_grouped(host), outs):
            assert np.array_equal(C.cpu().double().numpy(), Cr)


# ---------------------------------------------------------------- FP8 groups

from oracle import fp8 as ofp8  # noqa: E402
from gemm_inputs import make_fp8_operands  # noqa: E402

F8_SHAPES = [(300, 280, 400), (1, 256, 128), (0, 64, 128), (513, 130, 144), (64, 700, 512),
             (256, 256, 16)]
F8_CODE = {"e4m3": _lib.GEMM_FP8_E4M3, "e5m2": _lib.GEMM_FP8_E5M2}


def _f8_problems(shapes, fa, fb, mode, block_m, dist, seed, out_dt):
    host, keep, probs = [], [], []
    for g, (M, N, K) in enumerate(shapes):
        A, B, sa, sb = make_fp8_operands(M, N, K, fa, fb, dist, seed=seed + g, mode=mode,
                                         block_m=block_m)
        host.append((A, B, sa, sb, K))
        Ad, Bd, sad, sbd = A.to(DEV), B.to(DEV), sa.to(DEV), sb.to(DEV)
        Cd = torch.full((M, N), float("nan"), dtype=TORCH_DT[out_dt], device=DEV)
        keep.append((Ad, Bd, sad, sbd, Cd))
        probs.append(_lib.GemmGroupProblemFP8(Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), None,
                                              sad.data_ptr(), sbd.data_ptr(), M, N, K,
                                              max(K, 1), max(K, 1), max(N, 1)))
    return host, keep, probs


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
@pytest.mark.parametrize("mode,block_m", [("tensor", 1), ("block", 1), ("block", 128)])
def test_grouped_fp8_every_element(fa, fb, mode, block_m):
    say("case grouped fp8 %s x %s %s/%d" % (fa, fb, mode, block_m))
    host, keep, probs = _f8_problems(F8_SHAPES, fa, fb, mode, block_m, "uniform", 60, "bf16")
    h = new_handle()
    s = torch.cuda.current_stream(DEV)
    st = _lib.gemm_run_grouped_fp8(h._h, F8_CODE[fa], F8_CODE[fb], probs, CODE["bf16"], mode,
                                   block_m, None, s.cuda_stream)
    s.synchronize()
    h.close()
    assert st == _lib.GEMM_OK
    for g, ((A, B, sa, sb, K), k) in enumerate(zip(host, keep)):
        Cr, S = ofp8.gemm(A, B, K=K, fmt_a=fa, fmt_b=fb, mode=mode, scale_a=sa, scale_b=sb,
                          block_m=block_m)
        check(k[4].float().cpu().double().numpy(), Cr, S, "bf16", "fp8 group %d" % g)


@pytest.mark.parametrize("mode,block_m", [("tensor", 1), ("block", 1), ("block", 128)])
def test_grouped_fp8_small_integers_bitwise_and_equal_to_single_launches(mode, block_m):
    say("case grouped fp8 int3 %s/%d" % (mode, block_m))
    host, keep, probs = _f8_problems(F8_SHAPES, "e4m3", "e5m2", mode, block_m, "int3", 70, "fp32")
    h = new_handle()
    s = torch.cuda.current_stream(DEV)
    st = _lib.gemm_run_grouped_fp8(h._h, F8_CODE["e4m3"], F8_CODE["e5m2"], probs, CODE["fp32"],
                                   mode, block_m, None, s.cuda_stream)
    s.synchronize()
    h.close()
    assert st == _lib.GEMM_OK
    h1 = new_handle("256x256x64_w8_pp2", 1)
    for g, ((A, B, sa, sb, K), (Ad, Bd, sad, sbd, Cd)) in enumerate(zip(host, keep)):
        Cr, _ = ofp8.gemm(A, B, K=K, fmt_a="e4m3", fmt_b="e5m2", mode=mode, scale_a=sa,
                          scale_b=sb, block_m=block_m)
        C = Cd.cpu().double().numpy()
        assert np.array_equal(C, Cr), g
        M, N = Cd.shape
        if M and N and K:
            C1 = torch.empty((M, N), dtype=torch.float32, device=DEV)
            sc = _lib.fp8_scales(mode, sad.data_ptr(), sbd.data_ptr(), block_m)
            h1.run_raw_fp8(F8_CODE["e4m3"], F8_CODE["e5m2"], Ad.data_ptr(), Bd.data_ptr(),
                           C1.data_ptr(), M, N, K, K, K, N, CODE["fp32"], sc, None, s.cuda_stream)
            s.synchronize()
            assert torch.equal(C1, Cd), g
    h1.close()


def test_grouped_fp8_with_epilogue_and_checks():
    shapes = [(300, 280, 256), (64, 512, 128)]
    say("case grouped fp8 epilogue")
    host, keep, probs = _f8_problems(shapes, "e4m3", "e4m3", "block", 1, "uniform", 80, "bf16")
    g = torch.Generator().manual_seed(5)
    biases = [(torch.rand(N, generator=g) * 2 - 1).float() for _, N, _ in shapes]
    bds = [b.to(DEV) for b in biases]
    for p, bd in zip(probs, bds):
        p.bias = bd.data_ptr()
    h = new_handle()
    s = torch.cuda.current_stream(DEV)
    epi = _lib.epilogue(0.5, 0.0, 0, "n", "relu")
    st = _lib.gemm_run_grouped_fp8(h._h, F8_CODE["e4m3"], F8_CODE["e4m3"], probs, CODE["bf16"],
                                   "block", 1, epi, s.cuda_stream)
    s.synchronize()
    assert st == _lib.GEMM_OK
    for (A, B, sa, sb, K), k, b in zip(host, keep, biases):
        Cr, S = ofp8.gemm(A, B, K=K, mode="block", scale_a=sa, scale_b=sb, block_m=1)
        Dr = oepi.apply(Cr, alpha=0.5, bias=b.numpy(), bias_along="n", act="relu")
        aS, t = oepi.scale_of(S, alpha=0.5, bias=b.numpy(), bias_along="n")
        check_epilogue(k[4].float().cpu().double().numpy(), Dr, aS, t, "bf16", "fp8 group epi")
    # argument checks: K % 16, a null scale, an unknown block_m, a 16-bit format
    bad = _lib.GemmGroupProblemFP8(*[getattr(probs[0], f) for f, _ in probs[0]._fields_])
    bad.K = 24
    assert _lib.gemm_run_grouped_fp8(h._h, 3, 3, [bad], 0, "block", 1, None,
                                     s.cuda_stream) == _lib.GEMM_ERR_UNSUPPORTED
    bad = _lib.GemmGroupProblemFP8(*[getattr(probs[0], f) for f, _ in probs[0]._fields_])
    bad.scale_a = None
    assert _lib.gemm_run_grouped_fp8(h._h, 3, 3, [bad], 0, "tensor", 1, None,
                                     s.cuda_stream) == _lib.GEMM_ERR_INVALID_ARG
    assert _lib.gemm_run_grouped_fp8(h._h, 3, 3, probs, 0, "block", 64, None,
                                     s.cuda_stream) == _lib.GEMM_ERR_INVALID_ARG
    assert _lib.gemm_run_grouped_fp8(h._h, 0, 3, probs, 0, "block", 1, None,
                                     s.cuda_stream) == _lib.GEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    h.close()
