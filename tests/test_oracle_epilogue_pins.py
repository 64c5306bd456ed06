"""Pins of the fused-epilogue oracle (oracle/epilogue.py) to things other than
itself (runs without a GPU): closed forms whose every term is exact, the axis
a bias vector runs along on a non-square output, the sign rule of ReLU, and
GELU against standard-normal table values of Phi printed to 16 digits.
A dropped term, a bias along the wrong axis, a swapped alpha/beta or a wrong
GELU constant fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import epilogue
from gemm_inputs import make_operands


def test_identity_epilogue_returns_the_product():
    A, B = make_operands(7, 9, 40, "bf16", "uniform", seed=3)
    C, _ = oracle.gemm_nt(A, B, in_dtype="bf16")
    assert np.array_equal(epilogue.apply(C), C)


def test_axpby_closed_form_on_all_ones():
    # all-ones operands give C = K exactly; alpha = 0.5, beta = 2, C_old = 3:
    # D = K/2 + 6, every term exact in binary64
    K = 96
    A, B = make_operands(4, 6, K, "bf16", "ones")
    C, _ = oracle.gemm_nt(A, B, in_dtype="bf16")
    D = epilogue.apply(C, C_old=np.full((4, 6), 3.0), alpha=0.5, beta=2.0)
    assert np.all(D == K / 2 + 6)


def test_alpha_and_beta_are_not_swapped():
    K = 10
    A, B = make_operands(2, 3, K, "bf16", "ones")
    C, _ = oracle.gemm_nt(A, B, in_dtype="bf16")
    D = epilogue.apply(C, C_old=np.full((2, 3), 100.0), alpha=3.0, beta=0.25)
    assert np.all(D == 3 * K + 25)


def test_bias_along_n_and_along_m_on_a_non_square_output():
    M, N, K = 3, 5, 8
    A, B = make_operands(M, N, K, "bf16", "ones")
    C, _ = oracle.gemm_nt(A, B, in_dtype="bf16")
    bn = np.arange(N, dtype=np.float32) * 10
    bm = np.arange(M, dtype=np.float32) * 100
    Dn = epilogue.apply(C, bias=bn, bias_along="n")
    Dm = epilogue.apply(C, bias=bm, bias_along="m")
    for i in range(M):
        for j in range(N):
            assert Dn[i, j] == K + 10 * j
            assert Dm[i, j] == K + 100 * i
    with pytest.raises(ValueError):
        epilogue.apply(C, bias=bm, bias_along="n")


def test_bias_is_taken_in_fp32():
    C = np.zeros((1, 1))
    D = epilogue.apply(C, bias=np.array([0.1], dtype=np.float64), bias_along="n")
    assert D[0, 0] == float(np.float32(0.1)) and D[0, 0] != 0.1


def test_relu_clamps_negatives_only():
    # rank-1 with signs: C[i, j] = u_i v_j K
    u = np.array([1.0, -1.0, 2.0])
    v = np.array([-1.0, 1.0, 0.5, -2.0])
    K = 4
    A = torch.tensor(np.outer(u, np.ones(K)), dtype=torch.bfloat16)
    B = torch.tensor(np.outer(v, np.ones(K)), dtype=torch.bfloat16)
    C, _ = oracle.gemm_nt(A, B, in_dtype="bf16")
    D = epilogue.apply(C, act="relu")
    want = np.maximum(np.outer(u, v) * K, 0.0)
    assert np.array_equal(D, want)
    assert np.any(C < 0) and np.all(D >= 0)


# Phi(x) of the standard normal distribution, table values
_PHI = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, 3.0: 0.9986501019683699,
        0.5: 0.6914624612740131}


@pytest.mark.parametrize("x", [0.5, 1.0, 2.0, 3.0])
def test_gelu_is_x_times_phi_of_x(x):
    for s in (1.0, -1.0):
        v = s * x
        phi = _PHI[x] if s > 0 else 1.0 - _PHI[x]
        D = epilogue.apply(np.array([[v]]), act="gelu")
        assert abs(D[0, 0] - v * phi) <= 4e-16 * max(1.0, abs(v)), (v, D[0, 0], v * phi)


def test_gelu_special_values():
    D = epilogue.apply(np.array([[0.0, 40.0, -40.0]]), act="gelu")
    assert D[0, 0] == 0.0
    assert D[0, 1] == 40.0
    assert D[0, 2] == 0.0 or abs(D[0, 2]) < 1e-300


def test_order_bias_before_activation():
    # act(alpha acc + bias): with acc = 1, bias = -3 ReLU gives 0 (not 1 - 3 or 1)
    D = epilogue.apply(np.array([[1.0]]), bias=np.array([-3.0], dtype=np.float32),
                       bias_along="n", act="relu")
    assert D[0, 0] == 0.0
    D = epilogue.apply(np.array([[-1.0]]), alpha=-2.0, bias=np.array([0.5], dtype=np.float32),
                       bias_along="n", act="relu")
    assert D[0, 0] == 2.5


def test_scale_terms():
    S = np.array([[2.0, 4.0]])
    aS, t = epilogue.scale_of(S, C_old=np.array([[-1.0, 3.0]]), alpha=-0.5, beta=2.0,
                              bias=np.array([1.0, -2.0], dtype=np.float32), bias_along="n")
    assert np.array_equal(aS, [[1.0, 2.0]])
    assert np.array_equal(t, [[3.0, 8.0]])
    assert math.isclose(float(aS.sum()), 3.0)
