"""Compile the HIP library (gfx950) in place: ``python -m dense_gemm_nt_amd.build``."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
# the host side and one translation unit per group of kernel instantiations,
# compiled in parallel and linked into one shared library
SOURCES = [os.path.join(CSRC, f) for f in (
    "gemm_nt.hip", "launch_tiles_a.hip", "launch_tiles_b.hip",
    "launch_pp2.hip", "launch_pp2_km.hip", "launch_pp2_mk.hip", "launch_pp2_mm.hip",
    "launch_pp2_f8_e4e4.hip", "launch_pp2_f8_e4e5.hip", "launch_pp2_f8_e5e4.hip",
    "launch_pp2_f8_e5e5.hip", "launch_pp2_grouped.hip", "launch_pp2_persistent.hip", "launch_w4.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("gemm_nt_common.hpp", "gemm_nt_kernel.hpp",
                                           "gemm_nt_pp2.hpp", "gemm_nt_w4.hpp", "gemm_nt_trace.hpp",
                                           "gemm_nt_launch.hpp", "launch_pp2.hip",
                                           "launch_pp2_f8.hip", "launch_tiles_a.hip")] + \
    [os.path.join(ROOT, "include", "gemm_nt.h")]
LIB = os.path.join(PKG, "libgemm_nt.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
            # packed FP32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def command(out: str, extra=()) -> list:
    """One hipcc line that compiles and links every source (used by tools that
    want a single command, e.g. with extra -R remarks)."""
    return [hipcc(), *flags(), "-shared", *extra, *SOURCES, "-o", out]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False, jobs: int = 0, out: str = LIB, defines=()) -> str:
    """Compile every source and link them into `out` (the library by default;
    `defines` are extra -D flags, e.g. for an instrumented copy)."""
    tmpdir = tempfile.mkdtemp(prefix="gemm_nt_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        cmds = [[hipcc(), *flags(), *defines, "-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
        jobs = jobs or max(1, min(len(cmds), os.cpu_count() or 1, 8))
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            list(ex.map(_run, cmds))
        tmp = out + ".tmp%d" % os.getpid()
        link = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        _run(link)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
