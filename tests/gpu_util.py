"""Helpers for the GPU parity tests: run the HIP path through the C ABI on inputs
from gemm_inputs, and compare with the oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
from tests.tolerance import check

TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
CODE = {"bf16": 0, "fp16": 1, "fp32": 2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def new_handle(config=None, splits=None, persistent=False, streamk=None, inreduce=None, rotate=None):
    """A fresh library handle; `config` / `splits` force the plan for this handle,
    `persistent` runs its ping-pong tiles with persistent blocks, `streamk`
    (0 / 1 / 2) sets its stream-K mode (default: the plan rule), `inreduce`
    (0 / 1) the in-kernel reduction of two K splits (default: on), `rotate`
    (0 / 1 / 2) the k-slab order (natural, the M <= 128 rule (default), rotated)."""
    from dense_gemm_nt_amd import Gemm
    old = {k: os.environ.get(k) for k in ("GEMM_CONFIG", "GEMM_SPLITS", "GEMM_PERSIST", "GEMM_STREAMK",
                                          "GEMM_INREDUCE", "GEMM_ROTATE")}
    try:
        if rotate is not None:
            os.environ["GEMM_ROTATE"] = str(rotate)
        else:
            os.environ.pop("GEMM_ROTATE", None)
        if inreduce is not None:
            os.environ["GEMM_INREDUCE"] = str(inreduce)
        else:
            os.environ.pop("GEMM_INREDUCE", None)
        if streamk is not None:
            os.environ["GEMM_STREAMK"] = str(streamk)
        else:
            os.environ.pop("GEMM_STREAMK", None)
        if config:
            os.environ["GEMM_CONFIG"] = config
        else:
            os.environ.pop("GEMM_CONFIG", None)
        if splits:
            os.environ["GEMM_SPLITS"] = str(splits)
        else:
            os.environ.pop("GEMM_SPLITS", None)
        if persistent:
            os.environ["GEMM_PERSIST"] = "1"
        else:
            os.environ.pop("GEMM_PERSIST", None)
        return Gemm()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def run_gpu(h, A_store, B_store, K, in_dt, out_dt, ldc=None, stream=None, keep_device=False):
    """C = A[:, :K] . B[:, :K]^T on the GPU.  Returns the [M, N] result as float64
    numpy (or the device tensor with keep_device).  Columns of C beyond N (ldc > N)
    are filled with a sentinel first and must come back untouched."""
    M, lda = A_store.shape
    N, ldb = B_store.shape
    ldc = N if ldc is None else ldc
    dev = torch.device("cuda", 0)
    Ad = A_store.to(dev)
    Bd = B_store.to(dev)
    Cd = torch.full((max(M, 1), max(ldc, 1)), float("nan"), dtype=TORCH_DT[out_dt], device=dev)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    with torch.cuda.stream(s):
        h.run_raw(Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), M, N, K, lda, ldb, ldc,
                  CODE[in_dt], CODE[out_dt], s.cuda_stream)
    s.synchronize()
    if ldc > N and M > 0:
        assert bool(torch.isnan(Cd[:M, N:ldc].float()).all()), "kernel wrote past column N-1"
    if keep_device:
        return Cd[:M, :N]
    return Cd[:M, :N].float().cpu().to(torch.float64).numpy()


def compare_full(C, A_store, B_store, K, in_dt, out_dt, what):
    Cr, S = oracle.gemm_nt(A_store, B_store, K=K, in_dtype=in_dt)
    return check(C, Cr, S, out_dt, what)


def compare_sampled(C, A_store, B_store, K, in_dt, out_dt, what, n_rows=4, n_points=4000, seed=0):
    """Oracle on a few whole rows (first, last, random) and on random points."""
    M, N = C.shape
    rng = np.random.default_rng(seed)
    rows = sorted(set([0, M - 1] + list(rng.integers(0, M, max(0, n_rows - 2)))))
    Cr, S = oracle.gemm_nt_rows(A_store, B_store, rows, K=K, in_dtype=in_dt)
    r1 = check(C[rows], Cr, S, out_dt, what + " rows")
    ii = rng.integers(0, M, n_points)
    jj = rng.integers(0, N, n_points)
    Cp, Sp = oracle.gemm_nt_points(A_store, B_store, ii, jj, K=K, in_dtype=in_dt)
    r2 = check(C[ii, jj], Cp, Sp, out_dt, what + " points")
    return max(r1[0], r2[0]), max(r1[1], r2[1])
