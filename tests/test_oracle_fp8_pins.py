"""Pins of the FP8 oracle (oracle/fp8.py) to things other than itself, without
a GPU: every code of both formats against torch's float8 types, exact rational
sums on tiny blockwise cases, closed forms whose value depends on every block
index, and the agreement of constant block scales with per-tensor scaling.
A wrong exponent bias, a NaN/inf rule, a scale applied to the wrong k-block,
n-block or row block, or a transposed scale array fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8
from gemm_inputs import make_fp8_operands

TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_every_code_against_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes.copy()).view(TORCH[fmt]).to(torch.float64).numpy()
    got = fp8.decode(codes, fmt)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_format_landmarks():
    # E4M3: largest finite 448, no infinities; E5M2: largest finite 57344, +-inf
    e4 = fp8.decode(np.arange(256, dtype=np.uint8), "e4m3")
    e5 = fp8.decode(np.arange(256, dtype=np.uint8), "e5m2")
    assert np.nanmax(e4) == 448.0 and not np.any(np.isinf(e4))
    assert np.nanmax(e5[np.isfinite(e5)]) == 57344.0
    assert np.sum(np.isinf(e5)) == 2 and np.sum(np.isnan(e4)) == 2
    assert e4[0x01] == 2.0 ** -9 and e5[0x01] == 2.0 ** -16     # smallest subnormals


def _exact(A, B, K, fa, fb, mode, sa, sb, block_m):
    """Exact rational C via torch's own FP8 widening and Fractions."""
    a = torch.from_numpy(A.numpy().copy()).view(TORCH[fa]).to(torch.float64).numpy()
    b = torch.from_numpy(B.numpy().copy()).view(TORCH[fb]).to(torch.float64).numpy()
    M, N = a.shape[0], b.shape[0]
    sa, sb = sa.numpy(), sb.numpy()
    C = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            for k in range(K):
                if mode == "tensor":
                    s = Fraction(float(sa[0])) * Fraction(float(sb[0]))
                else:
                    s = Fraction(float(sa[i // block_m, k // 128])) * \
                        Fraction(float(sb[j // 128, k // 128]))
                t = Fraction(float(a[i, k])) * Fraction(float(b[j, k])) * s
                C[i][j] += t
                S[i][j] += abs(t)
    return C, S


@pytest.mark.parametrize("fa,fb,mode,block_m", [("e4m3", "e4m3", "block", 1),
                                                ("e5m2", "e4m3", "block", 128),
                                                ("e4m3", "e5m2", "tensor", 1)])
def test_exact_rationals_on_tiny_cases(fa, fb, mode, block_m):
    # N = 130 spans two 128-column scale blocks; K = 272 is two whole 128-deep
    # blocks and a ragged third; M = 130 spans two 128-row blocks
    M, N, K = (3, 130, 272) if block_m == 1 else (130, 3, 272)
    A, B, sa, sb = make_fp8_operands(M, N, K, fa, fb, "uniform", seed=4, mode=mode,
                                     block_m=block_m)
    C, S = fp8.gemm(A, B, K=K, fmt_a=fa, fmt_b=fb, mode=mode, scale_a=sa, scale_b=sb,
                    block_m=block_m)
    rows = range(M) if M <= 3 else [0, 127, 128, 129]
    cols = range(N) if N <= 3 else [0, 1, 127, 128, 129]
    # exact values element by element; each call sees one row and one column
    # with that row's and column's own block scales
    for i in rows:
        for j in cols:
            sai = sa[i // block_m:i // block_m + 1] if mode == "block" else sa
            sbj = sb[j // 128:j // 128 + 1] if mode == "block" else sb
            Ce, Se = _exact(A[i:i + 1], B[j:j + 1], K, fa, fb, mode, sai, sbj, block_m)
            tol = Fraction(K) * Fraction(2) ** -52 * Se[0][0]
            assert abs(Fraction(C[i, j]) - Ce[0][0]) <= tol
            assert abs(Fraction(S[i, j]) - Se[0][0]) <= tol


def test_closed_form_depends_on_every_block_index():
    # all codes 1.0 (E4M3 0x38); sa[i // 128][kb] = 2^kb * (1 + i // 128),
    # sb[j // 128][kb] = 3^(j // 128); K = 300 gives blocks of 128, 128, 44:
    # C[i, j] = (1 + i // 128) * 3^(j // 128) * (128 + 2 * 128 + 4 * 44)
    M, N, K = 200, 260, 300
    A = torch.full((M, K), 0x38, dtype=torch.uint8)
    B = torch.full((N, K), 0x38, dtype=torch.uint8)
    sa = torch.tensor([[2.0 ** kb * (1 + rb) for kb in range(3)] for rb in range(2)])
    sb = torch.tensor([[3.0 ** nb] * 3 for nb in range(3)])
    C, S = fp8.gemm(A, B, K=K, mode="block", scale_a=sa, scale_b=sb, block_m=128)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    want = (1 + ii // 128) * 3.0 ** (jj // 128) * (128 + 256 + 4 * 44)
    assert np.array_equal(C, want)
    assert np.array_equal(S, want)
    # per-row scales (block_m = 1) with a distinct value for every row
    sa1 = torch.tensor([[float(i + 1)] * 3 for i in range(M)])
    C1, _ = fp8.gemm(A, B, K=K, mode="block", scale_a=sa1, scale_b=torch.ones(3, 3),
                     block_m=1)
    assert np.array_equal(C1, (ii + 1) * float(K))


def test_constant_block_scales_equal_per_tensor_scaling():
    M, N, K = 40, 150, 256
    A, B, _, _ = make_fp8_operands(M, N, K, "e4m3", "e4m3", "uniform", seed=9)
    C1, _ = fp8.gemm(A, B, K=K, mode="tensor", scale_a=0.375, scale_b=1.5)
    C2, _ = fp8.gemm(A, B, K=K, mode="block", scale_a=torch.full((M, 2), 0.375),
                     scale_b=torch.full((2, 2), 1.5), block_m=1)
    assert np.array_equal(C1, C2)


def test_scale_array_shapes_are_checked():
    A, B, sa, sb = make_fp8_operands(4, 6, 256, mode="block", block_m=1)
    with pytest.raises(ValueError):
        fp8.gemm(A, B, K=256, mode="block", scale_a=sa.t().contiguous(), scale_b=sb)
    with pytest.raises(ValueError):
        fp8.gemm(A, B, K=256, mode="block", scale_a=sa, scale_b=sb, block_m=64)


def test_int3_recipe_is_exact_small_integers_and_powers_of_two():
    A, B, sa, sb = make_fp8_operands(130, 140, 384, "e5m2", "e4m3", "int3", seed=2,
                                     mode="block", block_m=128)
    a = fp8.decode(A, "e5m2")
    b = fp8.decode(B, "e4m3")
    assert set(np.unique(a)) <= set(range(-3, 4)) and set(np.unique(b)) <= set(range(-3, 4))
    for s in (sa, sb):
        e = np.log2(s.numpy())
        assert np.array_equal(e, np.round(e))


def _check_points(points_fn, fa, fb, mode, block_m):
    # fp8.gemm_points is the checker of the full-size FP8 tests: at every point
    # it equals fp8.gemm within the binary64 summation bound K 2^-53 S (the two
    # sum in different orders), and, at a few points, the exact rational sum.
    # M, N span two row blocks and two column blocks, K a ragged third k-block.
    M, N, K = 140, 131, 272
    A, B, sa, sb = make_fp8_operands(M, N, K, fa, fb, "uniform", seed=6, mode=mode,
                                     block_m=block_m)
    C, S = fp8.gemm(A, B, K=K, fmt_a=fa, fmt_b=fb, mode=mode, scale_a=sa, scale_b=sb,
                    block_m=block_m)
    rng = np.random.default_rng(3)
    ii = np.concatenate([rng.integers(0, M, 300), [0, 139, 5, 130, 130, 5]])
    jj = np.concatenate([rng.integers(0, N, 300), [130, 0, 130, 5, 127, 127]])
    Cp, Sp = points_fn(A, B, ii, jj, K=K, fmt_a=fa, fmt_b=fb, mode=mode, scale_a=sa,
                       scale_b=sb, block_m=block_m, chunk=64)
    bound = K * 2.0 ** -53 * S[ii, jj]
    assert np.all(np.abs(Cp - C[ii, jj]) <= bound)
    assert np.all(np.abs(Sp - S[ii, jj]) <= bound)
    for i, j, c in zip(ii[-6:], jj[-6:], Cp[-6:]):
        sai = sa[i // block_m:i // block_m + 1] if mode == "block" else sa
        sbj = sb[j // 128:j // 128 + 1] if mode == "block" else sb
        Ce, Se = _exact(A[i:i + 1], B[j:j + 1], K, fa, fb, mode, sai, sbj, block_m)
        assert abs(Fraction(float(c)) - Ce[0][0]) <= Fraction(K) * Fraction(2) ** -52 * Se[0][0]


@pytest.mark.parametrize("fa,fb,mode,block_m", [("e4m3", "e4m3", "tensor", 1),
                                                ("e4m3", "e4m3", "block", 1),
                                                ("e5m2", "e4m3", "block", 128),
                                                ("e4m3", "e5m2", "block", 1)])
def test_points_agree_with_full_product(fa, fb, mode, block_m):
    _check_points(fp8.gemm_points, fa, fb, mode, block_m)


def _swapped_points(A, B, ii, jj, **kw):
    return fp8.gemm_points(A, B, jj, ii, **kw)


def _swapped_formats(A, B, ii, jj, fmt_a, fmt_b, **kw):
    return fp8.gemm_points(A, B, ii, jj, fmt_a=fmt_b, fmt_b=fmt_a, **kw)


def _wrong_block_rows(A, B, ii, jj, block_m, **kw):
    return fp8.gemm_points(A, B, ii, jj, block_m=128 if block_m == 1 else 1, **kw)


@pytest.mark.parametrize("mutant", [_swapped_points, _swapped_formats, _wrong_block_rows])
def test_points_pin_catches_planted_mistakes(mutant):
    # exchanged coordinates, exchanged operand formats, or the other row-block
    # size of A's scales: each fails the pin above (a shape error counts too)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _check_points(mutant, "e5m2", "e4m3", "block", 1)
