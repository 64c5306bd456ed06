"""Pins of the grouped-GEMM oracle (oracle.gemm_grouped), without a GPU: the
block identity of matrix products (groups that share B equal one product of
the row-stacked A), empty groups, and the independence of each group's result
from the other groups and from their order.
"""
import numpy as np
import torch

import oracle
from gemm_inputs import make_operands


def test_groups_sharing_b_equal_the_stacked_product():
    # [A_0; A_1; A_2] . B^T = [A_0 B^T; A_1 B^T; A_2 B^T]
    K, N = 96, 40
    parts = [make_operands(m, N, K, "bf16", "uniform", seed=10 + m)[0] for m in (3, 17, 8)]
    _, B = make_operands(1, N, K, "bf16", "uniform", seed=99)
    outs = oracle.gemm_grouped([(A, B, K) for A in parts])
    C, S = oracle.gemm_nt(torch.cat(parts, 0), B, in_dtype="bf16")
    assert np.array_equal(np.concatenate([c for c, _ in outs], 0), C)
    assert np.array_equal(np.concatenate([s for _, s in outs], 0), S)


def test_empty_groups_and_order():
    probs = [make_operands(m, n, k, "fp16", "uniform", seed=m + n + k) + (k,)
             for (m, n, k) in ((5, 7, 16), (0, 9, 32), (4, 0, 8), (6, 3, 40))]
    outs = oracle.gemm_grouped(probs, in_dtype="fp16")
    assert outs[1][0].shape == (0, 9) and outs[2][0].shape == (4, 0)
    rev = oracle.gemm_grouped(probs[::-1], in_dtype="fp16")[::-1]
    for (c1, s1), (c2, s2) in zip(outs, rev):
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_each_group_uses_its_own_operands():
    # two groups with all-ones operands of different K: C_g = K_g everywhere
    g0 = make_operands(3, 4, 24, "bf16", "ones") + (24,)
    g1 = make_operands(2, 5, 40, "bf16", "ones") + (40,)
    (c0, _), (c1, _) = oracle.gemm_grouped([g0, g1])
    assert np.all(c0 == 24) and np.all(c1 == 40)
