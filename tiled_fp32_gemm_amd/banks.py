"""LDS bank arithmetic: the model the kernels' LDS layouts were derived from.

The pages reason about shared memory as banks of 4-byte words, with
``bank = (byte_address / 4) mod banks`` ("Chapter 3: Shared memory in
detail", section 3.1; "Memory-bank mechanism and accelerated compute",
section on how an address falls into a bank).  Lanes that ask for different
words of one bank in the same cycle are served one after another; lanes that
ask for the very same word are served together (broadcast; "CUDA in depth
(4)", section on broadcast).  Wide accesses must be analysed per instruction
and per group of lanes served together ("Memory-bank mechanism and
accelerated compute", section on double and float4).

Here the model is parameterised by the bank count and by how many lanes one
cycle serves.  The pages' examples use 32 banks and 32 lanes; gfx950 has 64
banks of 4 bytes, and a 64-lane wave's access of w bytes per lane is served
in groups of 256 / w lanes (64 lanes for 32-bit, 32 for 64-bit, 16 for
128-bit accesses).  The layouts in ``csrc/`` are written so that every
group touches each bank at most once; the hardware counter
SQ_LDS_BANK_CONFLICT confirms it (it reads 0 on the product kernel).

``KERNEL_ACCESSES`` restates, for each LDS access of the kernels, which
bytes each lane touches; ``tests/test_banks.py`` checks them all.
"""
from __future__ import annotations

from math import gcd
from typing import Callable, Iterable, Sequence

GFX950_BANKS = 64
BANK_BYTES = 4


def bank(byte_address: int, banks: int = GFX950_BANKS, width: int = BANK_BYTES) -> int:
    """Bank of the word holding ``byte_address``."""
    return (byte_address // width) % banks


def lanes_per_cycle(bytes_per_lane: int, banks: int = GFX950_BANKS,
                    width: int = BANK_BYTES, wave: int = 64) -> int:
    """Lanes served together: as many as fill every bank once."""
    return max(1, min(wave, banks * width // bytes_per_lane))


def conflict_degree(lane_bytes: Sequence[Iterable[int]], banks: int = GFX950_BANKS,
                    width: int = BANK_BYTES, group: int | None = None) -> int:
    """Worst number of distinct words one bank must serve in one cycle.

    ``lane_bytes[l]`` lists the byte addresses lane l touches in one access
    (one for a 4-byte access, 16 for a 128-bit one).  Lanes are served in
    consecutive groups of ``group`` lanes (default: ``lanes_per_cycle``).
    1 means conflict-free; equal words count once (broadcast)."""
    per_lane = [sorted({a // width for a in addrs}) for addrs in lane_bytes]
    if group is None:
        nbytes = max((len(w) for w in per_lane), default=1) * width
        group = lanes_per_cycle(nbytes, banks, width, len(per_lane))
    worst = 0
    for g0 in range(0, len(per_lane), group):
        words: dict[int, set[int]] = {}
        for w_list in per_lane[g0:g0 + group]:
            for w in w_list:
                words.setdefault(w % banks, set()).add(w)
        worst = max(worst, max((len(v) for v in words.values()), default=0))
    return worst


def strided(stride_words: int, lanes: int = 32, base: int = 0) -> list[list[int]]:
    """Lane l reads the 4-byte word base + l * stride (byte addresses)."""
    return [[4 * (base + l * stride_words)] for l in range(lanes)]


def gcd_rule(stride_words: int, banks: int = 32) -> tuple[int, int]:
    """(banks touched, conflict degree) of a full-width strided scalar read:
    banks / gcd(stride, banks) and gcd(stride, banks)."""
    g = gcd(stride_words, banks)
    return banks // g, g


def vec(addr: int, nbytes: int) -> list[int]:
    return list(range(addr, addr + nbytes))


# ---------------------------------------------------------------------------
# The kernels' LDS accesses, one 64-lane wave instruction each (byte
# addresses relative to the stage base).  Parameters follow the kernels.

def direct_a_read(bm: int = 256, bk: int = 32, wm0: int = 0, i: int = 0,
                  sub: int = 0, e: int = 0) -> list[list[int]]:
    """MFMA A fragment read of the LDS-direct kernel (128-bit)."""
    cpr = bk // 4
    out = []
    for lane in range(64):
        li, lh = lane & 31, lane >> 5
        row = wm0 + 32 * i + li
        unit = (row // 16) * (16 * cpr) + 16 * (4 * sub + 2 * lh + e) + row % 16
        out.append(vec(16 * unit, 16))
    return out


def direct_b_read(bn: int = 256, wn0: int = 0, j: int = 0, sub: int = 0,
                  p: int = 0) -> list[list[int]]:
    """MFMA B fragment read of the LDS-direct kernel (32-bit)."""
    qb = bn // 4
    out = []
    for lane in range(64):
        li, lh = lane & 31, lane >> 5
        k = 16 * sub + 8 * lh + p
        col = wn0 + 32 * j + li
        q = (col >> 2) ^ (8 if (k & 8) else 0)
        out.append([16 * (k * qb + q) + 4 * (col & 3)])
    return out


def direct_load(unit0: int = 0) -> list[list[int]]:
    """A load-to-LDS instruction: lane l fills 16 bytes at 16 (unit0 + l)."""
    return [vec(16 * (unit0 + l), 16) for l in range(64)]


def reg_a_store(bk: int = 16, f0: int = 0) -> list[list[int]]:
    """Register-staged A slab store, As[row][bk + 4] (128-bit)."""
    cpr, ra = bk // 4, bk + 4
    out = []
    for lane in range(64):
        f = f0 + lane
        row = (f & 15) + (f // (16 * cpr)) * 16
        kq = (f >> 4) % cpr
        out.append(vec(4 * (row * ra + 4 * kq), 16))
    return out


def reg_a_read(bk: int = 16, wm0: int = 0, i: int = 0, u: int = 0,
               e: int = 0) -> list[list[int]]:
    """Register-staged MFMA A fragment read (128-bit)."""
    ra = bk + 4
    return [vec(4 * ((wm0 + 32 * i + (l & 31)) * ra + 16 * u + 8 * (l >> 5) + 4 * e), 16)
            for l in range(64)]


def reg_b_store(bn: int = 128, f0: int = 0) -> list[list[int]]:
    """Register-staged B slab store, Bs[k][bn + 4] (128-bit)."""
    rb = bn + 4
    out = []
    for lane in range(64):
        f = f0 + lane
        k, jq = f // (bn // 4), f % (bn // 4)
        out.append(vec(4 * (k * rb + 4 * jq), 16))
    return out


def reg_b_read(bn: int = 128, wn0: int = 0, j: int = 0, u: int = 0,
               p: int = 0) -> list[list[int]]:
    """Register-staged MFMA B fragment read (32-bit)."""
    rb = bn + 4
    return [[4 * ((16 * u + 8 * (l >> 5) + p) * rb + wn0 + 32 * j + (l & 31))]
            for l in range(64)]


def fma_a_store(e: int = 0, f0: int = 0) -> list[list[int]]:
    """FMA kernel: A transposed into As[16][132], one 32-bit store of four."""
    out = []
    for lane in range(64):
        f = f0 + lane
        row = (f & 15) + ((f >> 6) << 4)
        kq = (f >> 4) & 3
        out.append([4 * ((4 * kq + e) * 132 + row)])
    return out


def fma_a_read(k: int = 0, half: int = 0, wave: int = 0) -> list[list[int]]:
    """FMA kernel: a thread's four A rows at one k (128-bit, broadcast)."""
    return [vec(4 * (k * 132 + 64 * half + 4 * (4 * wave + (l >> 4))), 16)
            for l in range(64)]


def fma_b_read(k: int = 0, half: int = 0) -> list[list[int]]:
    """FMA kernel: a thread's four B columns at one k (128-bit)."""
    return [vec(4 * (k * 132 + 64 * half + 4 * (l & 15)), 16) for l in range(64)]


def transpose_unit(layout: str, r: int, c: int) -> int:
    """16-byte unit of tile group (r, c) in the transpose kernel's layouts
    (tiles of 64 rows by 32 units)."""
    if layout == "padded":
        return 33 * r + c
    if layout == "swizzled":
        return 32 * r + (c ^ (r >> 2))
    return 32 * r + c


def transpose_store(layout: str, q: int = 0, wave: int = 0) -> list[list[int]]:
    """Tile row store (128-bit): thread f writes group (f / 32, f % 32)."""
    out = []
    for lane in range(64):
        f = q * 256 + 64 * wave + lane
        out.append(vec(16 * transpose_unit(layout, f >> 5, f & 31), 16))
    return out


def transpose_gather(layout: str, e: int = 0, wave: int = 0,
                     bq: int = 0) -> list[list[int]]:
    """Block read (128-bit): thread b reads group (4 (b % 16) + e, b / 16)."""
    out = []
    for lane in range(64):
        b = 256 * bq + 64 * wave + lane
        out.append(vec(16 * transpose_unit(layout, 4 * (b & 15) + e, b >> 4), 16))
    return out


def ladder_a_store(layout: str, e: int = 0, s: int = 0,
                   wave: int = 0) -> list[list[int]]:
    """Ladder 8x8 kernel: A's k-major split store (32-bit), element e of the
    groups of slot s.  layout: "unpadded" As[16][128], "padded" As[16][132],
    "xor" As[16][128] with the row XORed by 16 ((k / 4) mod 4)."""
    ra = 132 if layout == "padded" else 128
    out = []
    for lane in range(64):
        f = s * 256 + 64 * wave + lane
        row, kq = (f & 15) + ((f >> 6) << 4), (f >> 4) & 3
        k = 4 * kq + e
        col = row ^ (16 * ((k >> 2) & 3)) if layout == "xor" else row
        out.append([4 * (k * ra + col)])
    return out


def ladder_b_store(layout: str, e: int = 0, s: int = 0,
                   wave: int = 0) -> list[list[int]]:
    """Ladder 8x8 kernel with B transposed: element e of group (k, jq) =
    (f / 32, f % 32) goes to Bs[4 jq + e][k] (32-bit): "cols" pitch 16,
    "cols_padded" pitch 17."""
    rb = 17 if layout == "cols_padded" else 16
    out = []
    for lane in range(64):
        f = s * 256 + 64 * wave + lane
        k, jq = f // 32, f % 32
        out.append([4 * ((4 * jq + e) * rb + k)])
    return out


def ladder_b_read(layout: str, k: int = 0, col: int = 0,
                  wave: int = 0) -> list[list[int]]:
    """Ladder 8x8 kernel with B transposed (32-bit read of column 4 tx + col
    at depth k): "cols" Bs[128][16], "cols_padded" Bs[128][17]."""
    rb = 17 if layout == "cols_padded" else 16
    return [[4 * ((4 * (lane & 15) + col) * rb + k)] for lane in range(64)]


KERNEL_ACCESSES: dict[str, Callable[[], list[list[int]]]] = {
    "transpose padded store": lambda: transpose_store("padded", q=1, wave=2),
    "transpose swizzled store": lambda: transpose_store("swizzled", q=2, wave=3),
    "transpose swizzled store, last round": lambda: transpose_store("swizzled", q=7, wave=3),
    "transpose swizzled gather": lambda: transpose_gather("swizzled", e=1, wave=2),
    "transpose swizzled gather, e = 3": lambda: transpose_gather("swizzled", e=3),
    "transpose swizzled gather, second block": lambda: transpose_gather("swizzled", e=2, wave=1, bq=1),
    "transpose naive store": lambda: transpose_store("naive"),
    "direct A fragment read": direct_a_read,
    "direct A fragment read, k group 1, block 1": lambda: direct_a_read(i=1, e=1, sub=1),
    "direct B fragment read": direct_b_read,
    "direct B fragment read, step 7, block 1": lambda: direct_b_read(j=1, p=7, sub=1),
    "direct B fragment read, 128 columns": lambda: direct_b_read(bn=128, wn0=64),
    "direct load to LDS": direct_load,
    "register A store": reg_a_store,
    "register A store, 32-deep slab": lambda: reg_a_store(bk=32, f0=64),
    "register A read": reg_a_read,
    "register A read, 32-deep slab": lambda: reg_a_read(bk=32, u=1, e=1),
    "register B store": reg_b_store,
    "register B read": reg_b_read,
    "register B read, 64 columns": lambda: reg_b_read(bn=64, p=3),
    "ladder A store, padded": lambda: ladder_a_store("padded", e=1, s=1, wave=2),
    "ladder A store, XOR": lambda: ladder_a_store("xor", e=3, s=0, wave=1),
    "ladder B transposed read, padded": lambda: ladder_b_read("cols_padded", k=5, col=2),
    "FMA A transposed store": fma_a_store,
    "FMA A transposed store, element 3": lambda: fma_a_store(e=3, f0=192),
    "FMA A read": fma_a_read,
    "FMA B read": fma_b_read,
}
