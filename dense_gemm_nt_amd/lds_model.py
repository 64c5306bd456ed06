"""Bank model of the LDS layouts the kernels use (host side, no GPU).

"A Blackwell GEMM by Hand in CuTe DSL: TMA, mbarriers, TMEM, and tcgen05",
section 6 (The swizzle), describes shared memory as banks of 4-byte words: the
lanes served together cost one pass per distinct word the busiest bank must
deliver (the same word for several lanes is a broadcast).  Its XOR swizzle moves
the 16-byte chunks of a 128-byte row by the row index modulo 8, so one logical
chunk column of eight rows lands in eight different bank groups.  The page
prints the pass counts and the chunk permutation for that example; the tests
reproduce them with `group_passes` and `page_swizzle`.

The kernels store each operand K-major, one LDS row per M or N index, and put
logical chunk c of row r at physical chunk c ^ key(r) (`ROW_KEYS`, by row
length).  Both keys depend on r mod 16 only: a direct-to-LDS load fills 16
rows (64-byte rows) or 8 rows (128-byte rows) with one fixed lane-to-chunk map,
and an MFMA operand read covers 32 rows, so any dependence on a higher row bit
would make the loading lane and the reading lane disagree about where a chunk
lives.  The tests check that, that the loads' lane-to-chunk map is a
permutation of each row, and the pass counts of the MFMA operand read (lane l
reads row l % 32 of a 32-row block, logical chunk 2 ks + l // 32) for 16 lanes
over 64 banks and 8 lanes over 32 banks.
"""
from __future__ import annotations

from collections import defaultdict

WORD = 4        # bytes per bank word
CHUNK = 16      # bytes per lane of a 128-bit access


def group_passes(addrs, banks=32, access=CHUNK) -> int:
    """Passes one group of lanes needs: each lane reads `access` bytes from its
    byte address; a bank delivers one word per pass."""
    wanted = defaultdict(set)                # bank -> distinct words asked of it
    for a in addrs:
        first = a // WORD
        for w in range(first, first + access // WORD):
            wanted[w % banks].add(w)
    return max((len(v) for v in wanted.values()), default=0)


def page_swizzle(addr: int) -> int:
    """The page's 128-byte swizzle: the chunk index inside a 128-byte row is
    XORed with the row index modulo 8 (bytes inside a chunk stay put)."""
    row, in_row = divmod(addr, 128)
    chunk, byte = divmod(in_row, CHUNK)
    return row * 128 + CHUNK * (chunk ^ (row % 8)) + byte


# The kernels' keys, by LDS row length in bytes (gemm_nt_common.hpp, row_key).
ROW_KEYS = {
    128: lambda r: (r & 7) ^ ((r >> 3) & 1),   # eight chunks; r and r + 8 differ too
    64: lambda r: (r >> 2) & 3,                # four chunks; (r / 4) mod 4
}


def kernel_offset(row: int, chunk: int, pitch: int = 128, key=None) -> int:
    """Byte offset of logical chunk `chunk` of row `row` in a kernel tile."""
    k = ROW_KEYS[pitch] if key is None else key
    return row * pitch + CHUNK * (chunk ^ k(row))


def operand_read(ks: int, row0: int, pitch: int = 128, key=None):
    """Byte offsets of the 64 lanes of one MFMA operand read: lane l reads row
    row0 + l % 32, logical chunk 2 ks + l // 32 (8 consecutive 16-bit k values)."""
    return [kernel_offset(row0 + l % 32, 2 * ks + l // 32, pitch, key) for l in range(64)]


def worst_read_passes(pitch: int = 128, banks: int = 64, lanes: int = 16, rows: int = 256,
                      key=None) -> int:
    """Largest pass count over every lane group, k-step and 32-row block of a
    `rows`-row tile."""
    steps = pitch // (2 * CHUNK)
    worst = 0
    for row0 in range(0, rows, 32):
        for ks in range(steps):
            a = operand_read(ks, row0, pitch, key)
            for g in range(0, 64, lanes):
                worst = max(worst, group_passes(a[g:g + lanes], banks))
    return worst


def load_map_is_permutation(pitch: int = 128, rows: int = 256, key=None) -> bool:
    """A direct-to-LDS load writes its lanes' 16-byte pieces contiguously; the
    lane filling physical chunk p of row r fetches logical chunk p ^ key(r).
    True when every row's logical chunks land exactly once."""
    n = pitch // CHUNK
    for r in range(rows):
        homes = sorted((kernel_offset(r, c, pitch, key) - r * pitch) // CHUNK for c in range(n))
        if homes != list(range(n)):
            return False
    return True


def key_period_16(pitch: int = 128, key=None) -> bool:
    """The key depends on the row modulo 16 only."""
    k = ROW_KEYS[pitch] if key is None else key
    return all(k(r) == k(r % 16) for r in range(1024))
