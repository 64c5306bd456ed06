"""Compile-time resources of every kernel in the built library (no device work).

The gfx950 code objects are taken out of the library's offload bundles and
their AMDGPU metadata note (msgpack) is read for each kernel: private segment
(scratch) bytes, VGPR/AGPR and spill counts, static LDS and the workgroup size.
The MFMA instructions of each kernel are counted in the disassembly of those
same code objects.

What is pinned:
- no kernel the planner can choose touches scratch or spills a VGPR;
- static LDS fits the 160 KB of a compute unit, and each kernel's registers fit
  the occupancy its LDS allows (waves per SIMD x unified VGPRs <= 512);
- each main-loop kernel holds exactly (MFMAs per k-slab per wave) x (loop
  copies the source spells out) MFMA instructions: a loop body the compiler
  duplicated or a slab it dropped changes the count.
"""
import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

LDS_BYTES = 160 * 1024
REGS_PER_SIMD_LANE = 512          # unified VGPR + AGPR file per SIMD lane
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


@pytest.fixture(scope="module")
def kernels():
    from dense_gemm_nt_amd import build
    if build.stale():
        build.build()
    return _read_kernels(build.LIB)


def _sections(elf: bytes):
    """Name -> (offset, size, type) of the sections of a little-endian ELF64 file."""
    assert elf[:4] == b"\x7fELF" and elf[4] == 2 and elf[5] == 1
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQIIQQ", elf, shoff + i * shentsize) for i in range(shnum)]
    stroff = hdrs[shstrndx][4]
    out = {}
    for h in hdrs:
        name_off, sh_type, off, size = h[0], h[1], h[4], h[5]
        end = elf.index(b"\0", stroff + name_off)
        out[elf[stroff + name_off:end].decode()] = (off, size, sh_type)
    return out


def _code_objects(lib_path):
    """The gfx950 code objects of every offload bundle in `.hip_fatbin`."""
    data = open(lib_path, "rb").read()
    off, size, _ = _sections(data)[".hip_fatbin"]
    fat = data[off:off + size]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    objs = []
    pos = fat.find(magic)
    while pos >= 0:
        p = pos + len(magic)
        n, = struct.unpack_from("<Q", fat, p)
        p += 8
        for _ in range(n):
            e_off, e_size, t_len = struct.unpack_from("<QQQ", fat, p)
            p += 24
            triple = fat[p:p + t_len].decode()
            p += t_len
            if triple.endswith("gfx950"):
                objs.append(fat[pos + e_off:pos + e_off + e_size])
        pos = fat.find(magic, pos + 1)
    return objs


def _metadata(co: bytes):
    """The msgpack AMDGPU metadata (note type 32, owner "AMDGPU") of a code object."""
    import msgpack
    for off, size, sh_type in _sections(co).values():
        if sh_type != 7:                     # SHT_NOTE
            continue
        p, end = off, off + size
        while p < end:
            namesz, descsz, ntype = struct.unpack_from("<III", co, p)
            p += 12
            name = co[p:p + namesz].rstrip(b"\0")
            p += (namesz + 3) & ~3
            desc = co[p:p + descsz]
            p += (descsz + 3) & ~3
            if name == b"AMDGPU" and ntype == 32:
                return msgpack.unpackb(desc, raw=False)
    raise AssertionError("no AMDGPU metadata note")


def _mfma_counts(co: bytes):
    counts = {}
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "co.o")
        open(path, "wb").write(co)
        out = subprocess.run([OBJDUMP, "-d", "--no-show-raw-insn", path], check=True,
                             capture_output=True, text=True).stdout
    name = None
    for line in out.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            name = m.group(1)
            counts.setdefault(name, 0)
        elif name and "v_mfma" in line:
            counts[name] += 1
    return counts


def _read_kernels(lib_path):
    kernels = {}
    have_objdump = os.path.exists(OBJDUMP) or shutil.which("llvm-objdump")
    for co in _code_objects(lib_path):
        md = _metadata(co)
        mfma = _mfma_counts(co) if have_objdump else {}
        for k in md["amdhsa.kernels"]:
            k = dict(k)
            k["mfma"] = mfma.get(k[".name"])
            kernels[k[".name"]] = k
    return kernels


def _args(name):
    """Template arguments of a mangled kernel name, in order (ints and bools)."""
    m = re.search(r"I(.*)EEvNS_10KernelArgsE", name)
    assert m, name
    return [int(v) for _, v in re.findall(r"L([ib])(\d+)E", m.group(1))]


def _family(name):
    for f in ("gemm_nt_kernel", "gemm_nt_pp2", "gemm_nt_w4", "splitk_sum", "streamk_sum"):
        if f in name:
            return f
    return None


def _persistent_tiles(name):
    """The opt-in persistent-block form of the ping-pong kernel (PS = 1)."""
    return _family(name) == "gemm_nt_pp2" and _args(name)[-1] == 1


def test_every_family_is_built(kernels):
    fams = {}
    for n in kernels:
        fams.setdefault(_family(n), []).append(n)
    assert None not in fams, fams.get(None)
    # tile kernels: 128x128 with 4 stages, 4 stages K-masked and 2 stages, and
    # 32x128; 2 in x 3 out types each, in the natural and the rotated k-slab order
    assert len(fams["gemm_nt_kernel"]) == 4 * 6 * 2
    assert sum(_args(n)[-1] for n in fams["gemm_nt_kernel"]) == 4 * 6
    # ping-pong: NT, three MN-major layouts, grouped, persistent (2 x 3 each);
    # stream-K (2); FP8: 4 type pairs x 2 scale modes x 3 out, plain and grouped
    assert len(fams["gemm_nt_pp2"]) == 6 * 6 + 2 + 4 * 2 * 3 * 2
    assert len(fams["gemm_nt_w4"]) == 6
    assert len(fams["splitk_sum"]) == 3 and len(fams["streamk_sum"]) == 3


def test_no_scratch_no_spills(kernels):
    for n, k in kernels.items():
        if _persistent_tiles(n):
            # opt-in (never planned): the tile loop keeps the epilogue's state
            # live across units; at most two dwords per lane
            assert k[".private_segment_fixed_size"] <= 8, (n, k[".private_segment_fixed_size"])
            continue
        assert k[".private_segment_fixed_size"] == 0, (n, k[".private_segment_fixed_size"])
        assert k[".vgpr_spill_count"] == 0, (n, k[".vgpr_spill_count"])
        assert not k[".uses_dynamic_stack"], n


def test_lds_and_register_budget(kernels):
    for n, k in kernels.items():
        lds = k[".group_segment_fixed_size"]
        assert lds <= LDS_BYTES, (n, lds)
        if lds == 0:
            continue
        blocks = LDS_BYTES // lds                       # blocks per compute unit
        waves = -(-k[".max_flat_workgroup_size"] // 64)
        per_simd = blocks * -(-waves // 4)
        assert per_simd * k[".vgpr_count"] <= REGS_PER_SIMD_LANE, (n, per_simd, k[".vgpr_count"])
    # the two-stage 128x128 tile is the one meant to run two blocks per unit
    two = [n for n in kernels if _family(n) == "gemm_nt_kernel" and _args(n)[5] == 2]
    assert len(two) == 2 * 6
    for n in two:
        assert LDS_BYTES // kernels[n][".group_segment_fixed_size"] >= 2, n


def _expected_mfma(name):
    a = _args(name)
    fam = _family(name)
    if fam == "gemm_nt_kernel":
        bm, bn, bk, wm, wn = a[:5]
        return (bm // wm // 32) * (bn // wn // 32) * (bk // 16) * 2      # one loop per B policy
    if fam == "gemm_nt_pp2":
        in_t, sc = a[0], a[4]
        per_slab = 2 * 4 * (4 if in_t < 2 else 2)     # 64 x 128 per wave; x16 or x64 k-steps
        # group 0's loop twice (two B load policies; blockwise FP8 once),
        # group 1's loop and its last slab after the loop
        return per_slab * (3 if (in_t >= 2 and sc == 1) else 4)
    if fam == "gemm_nt_w4":
        bn = a[2]
        return 4 * (bn // 64) * 4 * 2                 # 128 x BN/2 per wave, two loop copies
    return 0


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not installed")
def test_mfma_count_per_loop(kernels):
    for n, k in kernels.items():
        assert k["mfma"] == _expected_mfma(n), (n, k["mfma"], _expected_mfma(n))
