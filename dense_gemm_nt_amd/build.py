"""Compile the HIP library (gfx950) in place: ``python -m dense_gemm_nt_amd.build``."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "gemm_nt.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("gemm_nt_common.hpp", "gemm_nt_kernel.hpp",
                                           "gemm_nt_pingpong.hpp", "gemm_nt_pp2.hpp")] + \
    [os.path.join(ROOT, "include", "gemm_nt.h")]
LIB = os.path.join(PKG, "libgemm_nt.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out: str, extra=()) -> list:
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
            # packed FP32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", *extra, *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
