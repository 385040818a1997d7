"""The LDS bank model against the pages' worked examples, and every LDS
access of the kernels against the gfx950 geometry (CPU only)."""
from __future__ import annotations

import json
import os

import pytest

from tiled_fp32_gemm_amd import banks

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "bank_examples.json")))


def test_address_to_bank():
    g = GOLDEN["address_to_bank"]
    for off, b in g["byte_offset_to_bank"]:
        assert banks.bank(off, g["banks"]) == b


def test_four_accesses():
    g = GOLDEN["four_accesses"]
    for stride, degree in g["stride_to_degree"]:
        acc = banks.strided(stride, g["lanes"])
        assert banks.conflict_degree(acc, g["banks"], group=g["lanes"]) == degree


def test_gcd_rule_matches_the_model():
    g = GOLDEN["gcd_rule"]
    for s in g["strides"]:
        acc = banks.strided(s, 32)
        touched = len({banks.bank(a[0], 32) for a in acc})
        want_touched, want_degree = banks.gcd_rule(s, g["banks"])
        assert touched == want_touched
        assert banks.conflict_degree(acc, 32, group=32) == want_degree


def test_three_threads_and_stride_16():
    g = GOLDEN["three_threads"]
    acc = [[4 * w] for w in g["words"]]
    assert banks.conflict_degree(acc, g["banks"], group=32) == g["degree"]
    g = GOLDEN["stride_16_pitfall"]
    assert banks.conflict_degree(banks.strided(g["stride"], g["lanes"]), 32,
                                 group=32) == g["degree"]
    assert banks.conflict_degree(banks.strided(g["padded_stride"], g["lanes"]),
                                 32, group=32) == g["padded_degree"]


def test_padding_residues():
    g = GOLDEN["padding_residues"]
    for idx, b in g["index_to_bank"]:
        assert banks.bank(4 * idx, g["banks"]) == b


def test_column_reads_of_a_tile():
    g = GOLDEN["column_read_32x32"]
    rows, cols = g["tile"]
    for col in (0, 5, 31):
        acc = [[4 * (r * cols + col)] for r in range(rows)]
        assert banks.conflict_degree(acc, 32, group=32) == g["degree"]
    rows, pcols = g["padded_tile"]
    for col in (0, 5, 31):
        acc = [[4 * (r * pcols + col)] for r in range(rows)]
        assert banks.conflict_degree(acc, 32, group=32) == g["padded_degree"]
        for r in range(rows):
            assert banks.bank(4 * (r * pcols + col), 32) == (r + col) % 32
    for r in range(rows):   # rows of the padded tile stay conflict-free too
        acc = [[4 * (r * pcols + c)] for c in range(32)]
        assert banks.conflict_degree(acc, 32, group=32) == 1


def test_xor_swizzle_is_a_permutation_both_ways():
    n = GOLDEN["xor_swizzle"]["tile"][0]
    for row in range(n):
        assert sorted(col ^ row for col in range(n)) == list(range(n))
    for col in range(n):
        assert sorted(col ^ row for row in range(n)) == list(range(n))
        acc = [[4 * (row * n + (col ^ row))] for row in range(n)]
        assert banks.conflict_degree(acc, 32, group=32) == 1


def test_tile_footprints():
    g = GOLDEN["tile_footprint_bytes"]
    assert 32 * 32 * 4 == g["tile_32x32"] and 32 * 33 * 4 == g["tile_32x33"]


def test_register_tile_traffic():
    for tm, tn, per_fma in GOLDEN["loads_per_fma"]["tiles"]:
        assert (tm + tn) / (tm * tn) == per_fma
    for T in GOLDEN["loads_per_tile_step"]["T"]:
        # T*T threads, T steps of k, one A and one B load each
        assert T * T * T * 2 == eval(GOLDEN["loads_per_tile_step"]["formula"])


def test_gfx950_lanes_per_cycle():
    assert banks.lanes_per_cycle(4) == 64
    assert banks.lanes_per_cycle(8) == 32
    assert banks.lanes_per_cycle(16) == 16
    assert banks.lanes_per_cycle(4, banks=32, wave=32) == 32


@pytest.mark.parametrize("name", sorted(banks.KERNEL_ACCESSES))
def test_kernel_lds_accesses_are_conflict_free_on_gfx950(name):
    acc = banks.KERNEL_ACCESSES[name]()
    assert len(acc) == 64
    assert banks.conflict_degree(acc, banks.GFX950_BANKS) == 1, name


def test_model_catches_a_bad_layout():
    # The unpadded 16-float A row (64-byte pitch) would make 16 consecutive
    # rows of one 128-bit fragment read share banks on gfx950: 4-way.
    acc = [banks.vec(4 * ((l & 31) * 16 + 8 * (l >> 5)), 16) for l in range(64)]
    assert banks.conflict_degree(acc, banks.GFX950_BANKS) == 4
    # and B read halves 8 rows apart with an unpadded 128-float pitch: 2-way
    acc = [[4 * ((8 * (l >> 5)) * 128 + (l & 31))] for l in range(64)]
    assert banks.conflict_degree(acc, banks.GFX950_BANKS) == 2


def test_transpose_gather_naive_and_padded_conflict():
    # the unpadded control: the 16 lanes of a 128-bit read share one bank
    # group; one extra unit per row leaves 4 distinct groups (4-way)
    for e in range(4):
        for w in range(4):
            for bq in range(2):
                kw = dict(e=e, wave=w, bq=bq)
                assert banks.conflict_degree(banks.transpose_gather("naive", **kw),
                                             banks.GFX950_BANKS) == 16
                assert banks.conflict_degree(banks.transpose_gather("padded", **kw),
                                             banks.GFX950_BANKS) == 4
                assert banks.conflict_degree(banks.transpose_gather("swizzled", **kw),
                                             banks.GFX950_BANKS) == 1


def test_ladder_layouts_conflict_as_designed():
    # the ladder's layout steps: A's split store 4-way without padding, free
    # with it or with the XOR swizzle; B read down a column 16-way when
    # transposed without padding, free with a 17-float pitch
    for e in range(4):
        for s in range(2):
            for w in range(4):
                kw = dict(e=e, s=s, wave=w)
                assert banks.conflict_degree(banks.ladder_a_store("unpadded", **kw)) == 4
                assert banks.conflict_degree(banks.ladder_a_store("padded", **kw)) == 1
                assert banks.conflict_degree(banks.ladder_a_store("xor", **kw)) == 1
    for k in range(16):
        for col in range(4):
            assert banks.conflict_degree(banks.ladder_b_read("cols", k=k, col=col)) == 16
            assert banks.conflict_degree(banks.ladder_b_read("cols_padded", k=k, col=col)) == 1
    # storing B transposed is a column walk too: a 16-float pitch puts a
    # row's 32 groups in one bank, 17 floats leaves 2 groups per bank (lanes
    # 16 groups apart, 16 * 4 * 17 floats = 68 * 16, a multiple of 64 apart)
    for e in range(4):
        for s in range(2):
            for w in range(4):
                kw = dict(e=e, s=s, wave=w)
                assert banks.conflict_degree(banks.ladder_b_store("cols", **kw)) == 32
                assert banks.conflict_degree(banks.ladder_b_store("cols_padded", **kw)) == 2
