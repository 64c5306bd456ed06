"""Bank model of the LDS tile layout the GEMM kernel uses (host-side, no GPU).

Model (from "A Blackwell GEMM by Hand in CuTe DSL: TMA, mbarriers, TMEM, and
tcgen05", section 6, The swizzle): memory is split into banks of 4-byte words;
a group of lanes is served in one pass when no bank has to deliver two different
words; the cost of a group is the largest number of distinct words one bank must
deliver.  A 128-byte XOR swizzle permutes the eight 16-byte chunks of a 128-byte
row by the row index, so the same logical chunk of consecutive rows lands in
different banks.  The page's own table (32 banks, 8 rows of 16 bytes) pins
`passes` and `sw128` here.

The kernel stores every operand tile K-major, one 128-byte row (64 16-bit values)
per M or N index, and puts logical chunk c of row r at physical chunk
c ^ key(r).  `KEY_MODES` lists the keys the kernel can be built with; the tests
show which of them give one pass per group for both 32-bank / 8-lane and
64-bank / 16-lane groupings of the MFMA operand read (64 lanes, lane l reads row
l % 32, chunk 2*ks + l // 32).
"""
from __future__ import annotations


def sw128(addr: int) -> int:
    """XOR address bits 7..9 (row within an 8-row period) into bits 4..6 (16-byte chunk)."""
    return addr ^ (((addr >> 7) & 0b111) << 4)


def passes(addrs, banks=32, word_bytes=4, access_bytes=16) -> int:
    """Largest number of distinct words any bank must serve for these accesses."""
    per_bank = {}
    for a in addrs:
        for w in range(access_bytes // word_bytes):
            word = a // word_bytes + w
            per_bank.setdefault(word % banks, set()).add(word)
    return max(len(s) for s in per_bank.values()) if per_bank else 0


# Row keys the kernel can use; the number is its template argument.
KEY_MODES = {
    0: lambda r: r & 7,                 # the 128-byte swizzle of the page
    1: lambda r: (r ^ (r >> 3)) & 7,    # also separates rows r and r+8
    2: lambda r: (r >> 1) & 7,          # pairs of rows share a key
}


def kernel_offset(row: int, chunk: int, mode: int, pitch: int = 128) -> int:
    """Byte offset of logical 16-byte chunk `chunk` of tile row `row`."""
    return row * pitch + 16 * (chunk ^ KEY_MODES[mode](row))


def fragment_read_addrs(ks: int, mode: int, row0: int = 0):
    """Byte offsets the 64 lanes of one MFMA operand read touch (rows row0..row0+31)."""
    return [kernel_offset(row0 + (l % 32), 2 * ks + l // 32, mode) for l in range(64)]


def read_passes(mode: int, banks: int, lanes_per_group: int) -> int:
    """Worst pass count over all lane groups, k-steps and 32-row blocks of a 256-row tile."""
    worst = 0
    for row0 in range(0, 256, 32):
        for ks in range(4):
            addrs = fragment_read_addrs(ks, mode, row0)
            for g in range(0, 64, lanes_per_group):
                worst = max(worst, passes(addrs[g:g + lanes_per_group], banks=banks))
    return worst


def dma_write_is_permutation(mode: int, rows: int = 256) -> bool:
    """Direct-to-LDS writes land lane-contiguously; each lane fetches the global chunk
    whose swizzled home is its slot.  True when that map is a bijection per row."""
    for r in range(rows):
        homes = sorted(kernel_offset(r, c, mode) - r * 128 for c in range(8))
        if homes != [16 * p for p in range(8)]:
            return False
    return True
