"""Pins of the oracle's operand layouts (oracle.logical_operand / oracle.gemm)
to things other than itself, without a GPU: the textbook product of numpy on
exact small integers for every layout pair, a hand-worked 3 x 2 example, a
pure-Python triple loop over storage offsets with padded leading dimensions, and
the transpose identity (A . B^T)^T = B . A^T.  An index exchanged on either
operand, a transpose applied to the wrong operand or a padding column read as
data fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_inputs import make_operands, make_stored, store

LAYOUTS = [("k", "mn"), ("mn", "k"), ("mn", "mn"), ("k", "k")]


def _ints(rows, cols, seed, dt=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-9, 10, (rows, cols), generator=g).to(dt)


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_matches_numpy_matmul_of_the_stored_arrays(la, lb):
    # Non-square M, N, K so that any exchanged index changes the shape or values;
    # products of integers below 10 in magnitude are exact in binary64.
    M, N, K = 5, 7, 3
    Xa = _ints(M, K, 1) if la == "k" else _ints(K, M, 1)
    Xb = _ints(N, K, 2) if lb == "k" else _ints(K, N, 2)
    a = Xa.double().numpy()
    b = Xb.double().numpy()
    # the textbook reading of each layout pair: C = op(A) @ op(B) with
    # op(A) = A or A^T, op(B)^T = B or B^T
    left = a if la == "k" else a.T
    right = b.T if lb == "k" else b
    want = left @ right
    got, S = oracle.gemm(Xa, Xb, la, lb, in_dtype="bf16")
    assert got.shape == (M, N)
    assert np.array_equal(got, want)
    assert np.array_equal(S, np.abs(left) @ np.abs(right))


def test_hand_worked_mn_major_a():
    # A stored MN-major as [K=2][M=3] = [[1, 2, 3], [4, 5, 6]] is the matrix
    # [[1, 4], [2, 5], [3, 6]]; with B = [[1, 0], [0, 1], [1, 1]] (K-major, N=3)
    # the product A . B^T is [[1, 4, 5], [2, 5, 7], [3, 6, 9]].
    Xa = torch.tensor([[1, 2, 3], [4, 5, 6]], dtype=torch.float16)
    Xb = torch.tensor([[1, 0], [0, 1], [1, 1]], dtype=torch.float16)
    C, _ = oracle.gemm(Xa, Xb, "mn", "k", in_dtype="fp16")
    assert C.tolist() == [[1, 4, 5], [2, 5, 7], [3, 6, 9]]
    # the same storage read K-major is a different (2 x 3) operand
    with pytest.raises(ValueError):
        oracle.gemm(Xa, Xb, "k", "k", in_dtype="fp16")


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_brute_force_over_storage_offsets_with_padding(la, lb):
    # (m, k) -> m * ld + k (K-major) or k * ld + m (MN-major) on the flat storage,
    # leading dimensions above the row length; padding holds NaN and must not
    # reach the result.
    M, N, K = 4, 6, 5
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=11)
    lda = (K if la == "k" else M) + 3
    ldb = (K if lb == "k" else N) + 2
    Xa, Xb = store(A, la, lda), store(B, lb, ldb)
    fa = Xa.double().numpy().ravel()
    fb = Xb.double().numpy().ravel()
    want = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            acc = 0.0
            for k in range(K):
                ai = fa[i * lda + k] if la == "k" else fa[k * lda + i]
                bj = fb[j * ldb + k] if lb == "k" else fb[k * ldb + j]
                acc += ai * bj
            want[i, j] = acc
    # the oracle sees the logical extents of the padded storage
    Va = Xa[:, :K] if la == "k" else Xa[:, :M]
    Vb = Xb[:, :K] if lb == "k" else Xb[:, :N]
    got, _ = oracle.gemm(Va, Vb, la, lb, in_dtype="bf16")
    assert np.all(np.isfinite(got))
    # products of two bf16 values are exact in binary64; the sums of five may
    # round differently in the two orders, by far less than this
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_transpose_identity():
    # (A . B^T)^T = B . A^T: swapping the operands and their layouts transposes C
    M, N, K = 9, 4, 13
    Xa, Xb = make_stored(M, N, K, "mn", "k", "fp16", "uniform", seed=5)
    C1, _ = oracle.gemm(Xa, Xb, "mn", "k", in_dtype="fp16")
    C2, _ = oracle.gemm(Xb, Xa, "k", "mn", in_dtype="fp16")
    assert np.array_equal(C1, C2.T)


def test_make_stored_keeps_the_values():
    M, N, K = 6, 5, 7
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=2)
    for la, lb in LAYOUTS:
        Xa, Xb = make_stored(M, N, K, la, lb, "bf16", "uniform", seed=2)
        assert torch.equal(torch.from_numpy(oracle.logical_operand(Xa, la).view(np.int16)),
                           A.view(torch.int16))
        assert torch.equal(torch.from_numpy(oracle.logical_operand(Xb, lb).view(np.int16)),
                           B.view(torch.int16))


def _storage_loop(Xa, Xb, la, lb, lda, ldb, i, j, K):
    """sum_k a(i, k) b(j, k) read straight from the flat storage offsets."""
    fa = Xa.double().numpy().ravel()
    fb = Xb.double().numpy().ravel()
    acc = 0.0
    for k in range(K):
        ai = fa[i * lda + k] if la == "k" else fa[k * lda + i]
        bj = fb[j * ldb + k] if lb == "k" else fb[k * ldb + j]
        acc += ai * bj
    return acc


def _check_points(points_fn, la, lb):
    # oracle.gemm_points is the checker of the full-size layout tests: at every
    # point it must equal oracle.gemm bitwise (same per-element sum) and the
    # plain loop over storage offsets.  M != N and points on both sides of the
    # diagonal, including (i, j) and (j, i) pairs, so exchanged coordinates or
    # operands change the values; padded leading dimensions hold NaN.
    M, N, K = 37, 23, 40
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=21)
    lda = (K if la == "k" else M) + 8
    ldb = (K if lb == "k" else N) + 8
    Xa, Xb = store(A, la, lda), store(B, lb, ldb)
    Va = Xa[:, :K] if la == "k" else Xa[:, :M]
    Vb = Xb[:, :K] if lb == "k" else Xb[:, :N]
    full, S = oracle.gemm(Va, Vb, la, lb, in_dtype="bf16")
    rng = np.random.default_rng(5)
    ii = list(rng.integers(0, M, 60)) + [0, M - 1, 3, 17, 17, 3]
    jj = list(rng.integers(0, N, 60)) + [N - 1, 0, 17, 3, 22, 22]
    Cp, Sp = points_fn(Va, Vb, ii, jj, la, lb, in_dtype="bf16")
    assert np.array_equal(Cp, full[ii, jj]) and np.array_equal(Sp, S[ii, jj])
    loop = np.array([_storage_loop(Xa, Xb, la, lb, lda, ldb, i, j, K) for i, j in zip(ii, jj)])
    assert np.allclose(Cp, loop, rtol=0, atol=1e-12)


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_points_agree_with_full_product_and_storage_loop(la, lb):
    _check_points(oracle.gemm_points, la, lb)


def _swapped_points(Va, Vb, ii, jj, la, lb, in_dtype):
    C, S = oracle.gemm_points(Va, Vb, jj, ii, la, lb, in_dtype=in_dtype)
    return C, S


def _swapped_layouts(Va, Vb, ii, jj, la, lb, in_dtype):
    return oracle.gemm_points(Va, Vb, ii, jj, lb, la, in_dtype=in_dtype)


@pytest.mark.parametrize("mutant", [_swapped_points, _swapped_layouts])
def test_points_pin_catches_planted_mistakes(mutant):
    # the pin above fails for a points function with exchanged coordinates or
    # exchanged operand layouts (an out-of-range index or a shape error counts
    # as failing); on the pair where the two layouts differ
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _check_points(mutant, "k", "mn")
