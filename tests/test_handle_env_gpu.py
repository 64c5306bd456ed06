"""Handle creation and the environment switches gemm_create reads, on the GPU
(gemm_create needs a current device): a failed workspace allocation comes back
as GEMM_ERR_ALLOC with no handle, an unknown GEMM_CONFIG as
GEMM_ERR_INVALID_ARG, and GEMM_LOG prints the plan gemm_plan reports."""
import ctypes
import os

import pytest
import torch

from gemm_inputs import make_operands
from tests.gpu_util import CODE, TORCH_DT, say

pytestmark = pytest.mark.gpu


class _env:
    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        for k, v in self.kv.items():
            os.environ[k] = v

    def __exit__(self, *exc):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _create():
    from dense_gemm_nt_amd import _lib
    torch.cuda.init()
    h = ctypes.c_void_p(12345)
    st = _lib.lib().gemm_create(ctypes.byref(h))
    return st, h


def test_failed_allocation_is_reported():
    from dense_gemm_nt_amd import _lib
    say("case gemm_create with GEMM_TEST_FAIL_ALLOC=1")
    with _env(GEMM_TEST_FAIL_ALLOC="1"):
        st, h = _create()
    assert _lib.STATUS[st] == "GEMM_ERR_ALLOC"
    assert h.value is None
    # the binding raises the status
    with _env(GEMM_TEST_FAIL_ALLOC="1"):
        with pytest.raises(_lib.GemmError) as e:
            _lib.gemm_create()
    assert _lib.STATUS[e.value.status] == "GEMM_ERR_ALLOC"
    # without the switch the same call succeeds
    st, h = _create()
    assert st == 0 and h.value
    assert _lib.lib().gemm_destroy(h) == 0


def test_unknown_config_is_rejected():
    from dense_gemm_nt_amd import _lib
    say("case gemm_create with an unknown GEMM_CONFIG")
    with _env(GEMM_CONFIG="64x64x32_nonexistent"):
        st, h = _create()
    assert _lib.STATUS[st] == "GEMM_ERR_INVALID_ARG" and h.value is None


def test_log_line_names_the_plan(capfd):
    from dense_gemm_nt_amd import _lib, Gemm
    M, N, K = 256, 10240, 8192
    say("case GEMM_LOG=1 M=%d N=%d K=%d" % (M, N, K))
    with _env(GEMM_LOG="1"):
        h = Gemm()
    dev = torch.device("cuda", 0)
    A, B = make_operands(M, N, K, "bf16", "llm", seed=1)
    Ad, Bd = A.to(dev), B.to(dev)
    Cd = torch.empty((M, N), dtype=TORCH_DT["bf16"], device=dev)
    capfd.readouterr()
    s = torch.cuda.current_stream(dev)
    h.run_raw(Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), M, N, K, K, K, N, CODE["bf16"],
              CODE["bf16"], s.cuda_stream)
    s.synchronize()
    err = capfd.readouterr().err
    h.close()
    plan = _lib.gemm_plan(M, N, K)
    lines = [ln for ln in err.splitlines() if ln.startswith("gemm_nt:")]
    assert len(lines) == 1, err
    ln = lines[0]
    assert "M=%d N=%d K=%d" % (M, N, K) in ln
    assert "cfg=%s" % plan["name"] in ln
    assert "splits=%d" % plan["splits"] in ln
    assert "grid=%d" % plan["workgroups"] in ln
