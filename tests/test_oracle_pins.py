"""Pins of the CPU oracle to things other than itself (runs without a GPU).

Each test states what fixes the expected value: exhaustive library conversions,
exact rational arithmetic, closed forms of the product, or a textbook library
routine.  A dropped term, a wrong index, a transposed operand, a wrong exponent
bias or a wrong rounding rule in the oracle fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from gemm_inputs import make_operands
from tests.tolerance import check, ulp


def _codes(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _exact_values(t):
    """Exact binary64 values of a 16-bit tensor via torch's own widening (independent of the oracle)."""
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------- decode tables

def test_decode_fp16_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = codes.view(np.float16).astype(np.float64)
    got = oracle.decode(codes, "fp16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_bf16_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode(codes, "bf16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


# ---------------------------------------------------------------- RNE encoding

def _encode_cases():
    g = torch.Generator().manual_seed(123)
    x = torch.randn(20000, generator=g, dtype=torch.float32) * torch.exp2(
        torch.randint(-30, 30, (20000,), generator=g).to(torch.float32))
    small = torch.rand(2000, generator=g) * 2 ** -13   # fp16 subnormal range
    big = torch.rand(500, generator=g) * 70000.0       # fp16 overflow boundary
    # exact ties of both formats: integers m + 0.5 ulp
    ties16 = torch.tensor([2049.0, 2051.0, 4097.0, 4099.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11,
                           65520.0, 65519.0, 2 ** -25, 3 * 2 ** -25], dtype=torch.float32)
    tiesbf = torch.tensor([257.0, 259.0, 261.0, 263.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                           -257.0, 4992.0 + 16.0, 5000.0], dtype=torch.float32)
    return torch.cat([x, small, -small, big, -big, ties16, tiesbf, torch.tensor([0.0, -0.0])])


@pytest.mark.parametrize("fmt,tdt", [("bf16", torch.bfloat16), ("fp16", torch.float16)])
def test_encode_rne_matches_library(fmt, tdt):
    x = _encode_cases()
    want = _codes(x.to(tdt))
    got = oracle.encode(x.to(torch.float64).numpy(), fmt)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def test_encode_known_codes():
    # values printed nowhere; fixed by the IEEE formats themselves
    assert int(oracle.encode([257.0], "bf16")[0]) == 0x4380    # tie 256|258 -> even 256
    assert int(oracle.encode([259.0], "bf16")[0]) == 0x4382    # tie 258|260 -> even 260
    assert int(oracle.encode([5000.0], "bf16")[0]) == 0x459C   # 5000 -> 4992
    assert int(oracle.encode([65520.0], "fp16")[0]) == 0x7C00  # rounds past max -> inf
    assert int(oracle.encode([65504.0], "fp16")[0]) == 0x7BFF


# ---------------------------------------------------------------- brute force

TINY = [(1, 1, 1), (1, 8, 3), (3, 5, 7), (8, 8, 8), (2, 3, 15), (7, 4, 16), (5, 6, 17),
        (4, 4, 33), (6, 2, 33)]


def _fraction_product(a_vals, b_vals):
    M, K = a_vals.shape
    N = b_vals.shape[0]
    C = [[None] * N for _ in range(M)]
    S = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            c = Fraction(0)
            s = Fraction(0)
            for k in range(K):
                p = Fraction(float(a_vals[i, k])) * Fraction(float(b_vals[j, k]))
                c += p
                s += abs(p)
            C[i][j] = c
            S[i][j] = s
    return C, S


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K", TINY)
def test_bruteforce_exact_rational(fmt, M, N, K):
    A, B = make_operands(M, N, K, fmt, "uniform", seed=M * 100 + N * 10 + K, lda=K + 8, ldb=K + 16)
    C, S = oracle.gemm_nt(A, B, K=K, in_dtype=fmt)
    Ce, Se = _fraction_product(_exact_values(A[:, :K]), _exact_values(B[:, :K]))
    for i in range(M):
        for j in range(N):
            # binary64 sequential sum of exact products: error <= (K-1) 2^-53 S
            bound = (K - 1) * 2.0 ** -53 * float(Se[i][j])
            assert abs(Fraction(C[i, j]) - Ce[i][j]) <= Fraction(bound), (i, j)
            assert abs(Fraction(S[i, j]) - Se[i][j]) <= Fraction(bound), (i, j)


@pytest.mark.parametrize("M,N,K", TINY)
def test_bruteforce_small_integers_bitwise(M, N, K):
    A, B = make_operands(M, N, K, "bf16", "int3", seed=7 + K, lda=K + 8)
    C, S = oracle.gemm_nt(A, B, K=K, in_dtype="bf16")
    Ce, Se = _fraction_product(_exact_values(A[:, :K]), _exact_values(B[:, :K]))
    for i in range(M):
        for j in range(N):
            assert Fraction(C[i, j]) == Ce[i][j]
            assert Fraction(S[i, j]) == Se[i][j]


def test_nan_padding_is_never_read():
    A, B = make_operands(9, 11, 40, "fp16", "uniform", seed=3, lda=56, ldb=48)
    C, S = oracle.gemm_nt(A, B, K=40, in_dtype="fp16")
    assert np.all(np.isfinite(C)) and np.all(np.isfinite(S))


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("K", [1, 17, 512, 5000])
def test_all_ones_gives_K(K):
    A, B = make_operands(3, 5, K, "bf16", "ones")
    C, S = oracle.gemm_nt(A, B, in_dtype="bf16")
    assert np.all(C == K) and np.all(S == K)


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_identity_B_gives_A(fmt):
    K = 37
    A, _ = make_operands(6, K, K, fmt, "uniform", seed=11)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    B = torch.eye(K, dtype=dt)
    C, S = oracle.gemm_nt(A, B, in_dtype=fmt)
    assert np.array_equal(C, _exact_values(A))
    assert np.array_equal(S, np.abs(_exact_values(A)))


def test_rank1_closed_form():
    # A[i,k] = u_i x_k, B[j,k] = v_j x_k with powers of two: C = u_i v_j sum_k x_k^2 exactly
    M, N, K = 5, 7, 300
    g = np.random.default_rng(5)
    u = 2.0 ** g.integers(-3, 4, M) * g.choice([-1, 1], M)
    v = 2.0 ** g.integers(-3, 4, N) * g.choice([-1, 1], N)
    x = 2.0 ** g.integers(-4, 3, K) * g.choice([-1, 1], K)
    A = torch.tensor(np.outer(u, x), dtype=torch.bfloat16)
    B = torch.tensor(np.outer(v, x), dtype=torch.bfloat16)
    C, S = oracle.gemm_nt(A, B, in_dtype="bf16")
    want = np.outer(u, v) * float(np.sum(x * x))
    assert np.array_equal(C, want)
    assert np.array_equal(S, np.abs(want))


def test_operand_order_is_A_times_B_transpose():
    # a non-square case where A.B^T, A^T.B and B.A^T all differ in shape or value
    A = torch.tensor([[1.0, 2.0, 3.0]], dtype=torch.bfloat16)           # 1 x 3
    B = torch.tensor([[1.0, 0.0, 0.0], [0.0, 0.0, 2.0]], dtype=torch.bfloat16)  # 2 x 3
    C, _ = oracle.gemm_nt(A, B, in_dtype="bf16")
    assert C.shape == (1, 2)
    assert C.tolist() == [[1.0, 6.0]]


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("fmt,dist", [("bf16", "uniform"), ("fp16", "uniform"), ("bf16", "llm")])
def test_matches_numpy_float64_matmul(fmt, dist):
    M, N, K = 37, 45, 300
    A, B = make_operands(M, N, K, fmt, dist, seed=2)
    C, S = oracle.gemm_nt(A, B, in_dtype=fmt)
    ref = _exact_values(A) @ _exact_values(B).T
    assert np.all(np.abs(C - ref) <= 2 * K * 2.0 ** -53 * S + 1e-300)
    assert np.allclose(S, np.abs(_exact_values(A)) @ np.abs(_exact_values(B)).T, rtol=1e-13, atol=0)


def test_rows_and_points_agree_bitwise_with_full():
    M, N, K = 20, 30, 100
    A, B = make_operands(M, N, K, "fp16", "uniform", seed=4, lda=104)
    C, S = oracle.gemm_nt(A, B, K=K, in_dtype="fp16")
    rows = [19, 0, 7]
    Cr, Sr = oracle.gemm_nt_rows(A, B, rows, K=K, in_dtype="fp16")
    assert np.array_equal(Cr, C[rows]) and np.array_equal(Sr, S[rows])
    ii, jj = [0, 19, 5, 5], [29, 0, 3, 4]
    Cp, Sp = oracle.gemm_nt_points(A, B, ii, jj, K=K, in_dtype="fp16")
    assert np.array_equal(Cp, C[ii, jj]) and np.array_equal(Sp, S[ii, jj])


def test_rejects_bad_arguments():
    A, B = make_operands(4, 4, 8, "bf16", "uniform")
    with pytest.raises(ValueError):
        oracle.gemm_nt(A, B, K=9)          # K beyond the stored columns
    with pytest.raises(ValueError):
        oracle.gemm_nt_rows(A, B, [4])     # row out of range


def test_empty_K_gives_zero():
    A = torch.zeros((3, 0), dtype=torch.bfloat16)
    B = torch.zeros((2, 0), dtype=torch.bfloat16)
    C, S = oracle.gemm_nt(A, B, K=0)
    assert C.shape == (3, 2) and np.all(C == 0) and np.all(S == 0)


# ---------------------------------------------------------------- acceptance check

def test_tolerance_check_accepts_exact_and_rejects_off_by_bound():
    ref = np.array([[1.0, 300.0, -2.0e-3]])
    S = np.array([[10.0, 300.0, 5.0]])
    check(ref, ref, S, "fp32")
    bad = ref.copy()
    bad[0, 1] += 1e-3 * 300.0 + 1e-5 + 1e-9
    with pytest.raises(AssertionError):
        check(bad, ref, S, "fp32")
    # a bf16 result one ulp off passes only with the ulp term
    one_ulp = ref.copy()
    one_ulp[0, 0] += float(ulp(np.array([1.0]), "bf16")[0])
    check(one_ulp, ref, np.zeros_like(S), "bf16")
    with pytest.raises(AssertionError):
        check(one_ulp, ref, np.zeros_like(S), "fp32")


def test_ulp_values():
    assert ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -7
    assert ulp(np.array([1.0]), "fp16")[0] == 2.0 ** -10
    assert ulp(np.array([300.0]), "bf16")[0] == 2.0
    assert ulp(np.array([0.0]), "fp16")[0] == 2.0 ** -24
    assert ulp(np.array([0.0]), "bf16")[0] == 2.0 ** -133


def test_input_generator_is_deterministic_and_ordered():
    A1, B1 = make_operands(8, 9, 10, "bf16", "uniform", seed=0)
    A2, B2 = make_operands(8, 9, 10, "bf16", "uniform", seed=0)
    assert torch.equal(A1, A2) and torch.equal(B1, B2)
    g = torch.Generator().manual_seed(0)
    a = (torch.rand((8, 10), generator=g) * 2 - 1).to(torch.bfloat16)
    assert torch.equal(A1, a)          # A is drawn first from the seeded stream
    A3, B3 = make_operands(8, 9, 10, "bf16", "llm", seed=0)
    assert float(B3.float().abs().max()) < 0.2 < float(A3.float().abs().max())
