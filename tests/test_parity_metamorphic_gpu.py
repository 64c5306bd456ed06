"""Metamorphic pins of the HIP path (through the C ABI), on the GPU.

"Matmul on sm_120", The tiled view: the tiled sum is the same sum as the
per-element definition, in another order.  What follows holds for any order the
kernels choose, so it is checked bitwise, not within a tolerance:

  * scaling A by 2^s scales every product and every partial sum by 2^s exactly
    (no overflow or underflow at these magnitudes), so the FP32 output of the
    same shape (same plan, same order) scales bitwise;
  * on small integers every partial sum is exact, so gemm(B, A) is gemm(A, B)
    transposed and a permutation of the rows of A (of B) permutes the rows
    (the columns) of C, bitwise;
  * permuting whole 256-row blocks of A on random values moves each output
    row to a position with the same offset inside its tile, so it keeps its
    summation order and its bits.

Each of these also catches an index mistake (a transposed operand, a tile
stored at the wrong place) that the oracle comparison would report as an
error bound violation.
"""
import numpy as np
import pytest
import torch

from gemm_inputs import make_operands
from tests.gpu_util import new_handle, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def h():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return new_handle()


def _scaled(X, s):
    # exact: a power of two times a 16-bit value stays representable here
    return (X.float() * 2.0 ** s).to(X.dtype)


# BF16 inputs only: their subnormals (below 2^-126) are out of reach of these
# values, while FP16 inputs include subnormals whose handling inside the MFMA
# the scaling would change.
@pytest.mark.parametrize("M,N,K,ind,dist", [(4096, 4096, 4096, "bf16", "uniform"),
                                            (256, 8192, 8192, "bf16", "llm"),
                                            (1000, 4097, 1536, "bf16", "uniform"),
                                            (3000, 3000, 5000, "bf16", "uniform"),
                                            (1, 8192, 8192, "bf16", "uniform")])
@pytest.mark.parametrize("s", [-3, 5])
def test_power_of_two_scaling_of_A_scales_C_bitwise(h, M, N, K, ind, dist, s):
    say("case 2^%d A M=%d N=%d K=%d %s %s" % (s, M, N, K, ind, dist))
    A, B = make_operands(M, N, K, ind, dist, seed=11)
    As = _scaled(A, s)
    assert torch.equal(As.float(), A.float() * 2.0 ** s)      # the scaling itself is exact
    C = run_gpu(h, A, B, K, ind, "fp32")
    Cs = run_gpu(h, As, B, K, ind, "fp32")
    assert np.array_equal(Cs, C * 2.0 ** s)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (256, 8192, 8192), (300, 2000, 1536),
                                   (1, 4096, 8192), (127, 5000, 4104)])
def test_swapped_operands_transpose_C_bitwise(h, M, N, K):
    say("case gemm(B, A) = gemm(A, B)^T M=%d N=%d K=%d" % (M, N, K))
    A, B = make_operands(M, N, K, "bf16", "int3", seed=M + K)
    C = run_gpu(h, A, B, K, "bf16", "fp32")
    Ct = run_gpu(h, B, A, K, "bf16", "fp32")
    assert np.array_equal(Ct, C.T)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (256, 10240, 8192), (1000, 4097, 1536)])
def test_row_and_column_permutations_bitwise(h, M, N, K):
    say("case permutation equivariance M=%d N=%d K=%d" % (M, N, K))
    A, B = make_operands(M, N, K, "bf16", "int3", seed=7)
    g = torch.Generator().manual_seed(M + N)
    pr, pc = torch.randperm(M, generator=g), torch.randperm(N, generator=g)
    C = run_gpu(h, A, B, K, "bf16", "fp32")
    Cr = run_gpu(h, A[pr].contiguous(), B, K, "bf16", "fp32")
    Cc = run_gpu(h, A, B[pc].contiguous(), K, "bf16", "fp32")
    assert np.array_equal(Cr, C[pr.numpy()])
    assert np.array_equal(Cc, C[:, pc.numpy()])


def test_tile_block_permutation_on_random_values_bitwise(h):
    M, N, K = 4096, 4096, 4096
    say("case 256-row block permutation, random values, M=%d N=%d K=%d" % (M, N, K))
    A, B = make_operands(M, N, K, "bf16", "uniform", seed=5)
    g = torch.Generator().manual_seed(1)
    blocks = torch.randperm(M // 256, generator=g)
    rows = (blocks[:, None] * 256 + torch.arange(256)[None, :]).reshape(-1)
    C = run_gpu(h, A, B, K, "bf16", "fp32")
    Cp = run_gpu(h, A[rows].contiguous(), B, K, "bf16", "fp32")
    assert np.array_equal(Cp, C[rows.numpy()])
