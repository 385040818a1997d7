"""Static count of LDS traffic in the built kernels' main loops (CPU only).

The pages count shared-memory loads per FMA: 2 for the one-output-per-thread
loop, (TM + TN) / (TM TN) for a TM x TN register tile ("CUDA in depth (4):
accessing shared memory efficiently", sections on too many shared-memory
reads and on going from 1x1 to 2x2).  Here the same count is read off the
gfx950 assembly of this library: words moved by LDS reads and multiply-adds
(or matrix instructions) issued in one trip of each kernel's K loop.
"""
from __future__ import annotations

import re
import shutil

import pytest

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None,
                                reason="needs hipcc to build the assembly")

READ_WORDS = {"ds_read_b32": 1, "ds_read2_b32": 2, "ds_read2st64_b32": 2,
              "ds_read_b64": 2, "ds_read2_b64": 4, "ds_read2st64_b64": 4,
              "ds_read_b96": 3, "ds_read_b128": 4}


@pytest.fixture(scope="module")
def asm():
    from tiled_fp32_gemm_amd import build
    return open(build.build_asm()).read()


def kernel_body(asm: str, *parts: str) -> str:
    names = [n for n in re.findall(r"^(_ZN2sg\w+):", asm, re.M)
             if all(p in n for p in parts)]
    assert len(names) == 1, (parts, names)
    start = asm.index(names[0] + ":")
    return asm[start:asm.index(".Lfunc_end", start)]


def blocks(body: str) -> list[tuple[str, str, list[str]]]:
    """(label, comment text, instructions) of each basic block."""
    out = []
    for line in body.split("\n"):
        m = re.match(r"^(\.LBB\w+|; %bb\.\d+):(.*)$", line)
        if m:
            out.append([m.group(1), m.group(2), []])
            continue
        s = line.strip()
        if not out or not s:
            continue
        if s.startswith(";"):
            if not out[-1][2]:          # comment lines right after the label
                out[-1][1] += " " + s
            continue
        if not s.startswith("."):
            out[-1][2].append(s.split()[0])
    return [tuple(b) for b in out]


def main_loop(body: str, depth: int = 1) -> list[str]:
    """Instructions of the blocks of the first loop at ``depth`` (its own
    blocks only, not those of loops nested in it)."""
    bl = blocks(body)
    hdr = next((b for b in bl if re.search(
        rf"=>\s*This (?:Inner )?Loop Header: Depth={depth}", b[1])), None)
    assert hdr, "no loop"
    tag = hdr[0][2:] if hdr[0].startswith(".L") else hdr[0]
    insts = []
    for label, comment, ins in bl:
        if label == hdr[0] or f"in Loop: Header={tag} Depth={depth}" in comment:
            insts += ins
    return insts


def counts(insts: list[str]) -> dict:
    return {
        "words": sum(READ_WORDS.get(i, 0) for i in insts),
        "mfma": sum(i.startswith("v_mfma_f32_32x32x2") for i in insts),
        "fma": sum(i in ("v_fma_f32", "v_fmac_f32", "v_fmac_f32_e32",
                         "v_fma_f32_e64") for i in insts),
        "other_reads": sorted({i for i in insts
                               if i.startswith("ds_read") and i not in READ_WORDS}),
    }


def test_simple_kernel_is_two_loads_per_fma(asm):
    c = counts(main_loop(kernel_body(asm, "sgemm_simple_kernel")))
    assert not c["other_reads"]
    assert c["fma"] == 16                 # one output, 16 k per tile step
    assert c["words"] / c["fma"] == 2.0   # the pages' 1x1 figure


@pytest.mark.parametrize("flags", ["Lb1ELb1ELb1E", "Lb0ELb0ELb0E"])
def test_fma_kernel_is_the_8x8_register_tile(asm, flags):
    body = kernel_body(asm, "sgemm_fma_kernel", flags)
    # the k loop of a slab is unrolled by 8, inside the loop over slabs
    c = counts(main_loop(body, depth=2))
    assert not c["other_reads"]
    assert c["fma"] == 8 * 64                    # 8 k x 8 x 8
    assert c["words"] / c["fma"] == (8 + 8) / (8 * 8)


# (template fragment, TA, TB, 16-deep sub-slabs per wave group per slab)
DIRECT = [("Li256ELi256ELi64ELi64ELi32ELi1E", 2, 2, 2),
          ("Li128ELi128ELi32ELi64ELi32ELi1E", 1, 2, 2),
          ("Li64ELi128ELi32ELi64ELi32ELi1E", 1, 2, 2),
          ("Li64ELi128ELi32ELi64ELi32ELi2E", 1, 2, 1),
          ("Li64ELi64ELi32ELi32ELi32ELi1E", 1, 1, 2),
          ("Li64ELi64ELi32ELi32ELi32ELi2E", 1, 1, 1),
          ("Li32ELi64ELi32ELi32ELi32ELi2E", 1, 1, 1),
          ("Li32ELi64ELi32ELi32ELi64ELi4E", 1, 1, 1)]


@pytest.mark.parametrize("split", ["Lb0E", "Lb1E"])
@pytest.mark.parametrize("frag,ta,tb,subs", DIRECT, ids=[d[0] for d in DIRECT])
def test_direct_kernel_lds_traffic(asm, frag, ta, tb, subs, split):
    # the same main loop with and without K split across workgroups
    # (two LDS stages: the Li2E before the split flag)
    c = counts(main_loop(kernel_body(asm, "sgemm_mfma_direct_kernel", frag + "Li2E" + split)))
    assert not c["other_reads"]
    # per 16-deep sub-slab: 8 steps of TA x TB matrix instructions, fed by
    # two 128-bit A reads per 32-row block and eight B words per 32 columns
    assert c["mfma"] == subs * 8 * ta * tb
    assert c["words"] == subs * 8 * (ta + tb)
    # LDS bytes per flop of the wave: 64 lanes x 4 B per word over 4096
    # flops per 32x32x2 instruction
    assert c["words"] * 4 * 64 / (c["mfma"] * 4096) == (ta + tb) / (16 * ta * tb)


@pytest.mark.parametrize("tm,layout", [(1, "1ELi0"), (2, "1ELi0"), (4, "1ELi0"),
                                       (8, "1ELi0"), (8, "1ELi1"), (8, "0ELi0")])
def test_ladder_register_tiles_cut_lds_reads(asm, tm, layout):
    """The ladder's TM x TM register tiles: LDS words read per multiply-add
    equal (TM + TN) / (TM TN) -- 2, 1, 0.5 and 0.25 for 1x1 ... 8x8, in
    whatever layout A and B take."""
    body = kernel_body(asm, "sgemm_ladder_kernel", f"ILi{tm}ELi{tm}ELi{layout}ELb0E")
    words = sum(READ_WORDS.get(i.split()[0], 0) for i in re.findall(
        r"^\s+(ds_read\S*)", body, re.M))
    fmas = len(re.findall(r"^\s+v_fmac?_f32(?:_e32|_e64)?\s", body, re.M))
    assert fmas > 0
    assert words / fmas == pytest.approx((tm + tm) / (tm * tm)), (words, fmas)


@pytest.mark.parametrize("frag,ta,tb,subs", DIRECT, ids=[d[0] for d in DIRECT])
def test_direct_kernel_c_stores(asm, frag, ta, tb, subs):
    """The epilogue's stores: with one 32-column block per wave, one 32-bit
    store per accumulator element (TA blocks of 16 per lane); with two, whose
    columns interleave, one 64-bit store per pair of elements, and in the
    separate path of a tile on C's right edge one 32-bit store per element.
    A product's C goes out with the nontemporal hint, the split partials,
    which the reduction reads straight back, without it."""
    want = ({"buffer_store_dword": ta * 16} if tb == 1 else
            {"buffer_store_dwordx2": ta * 16, "buffer_store_dword": 2 * ta * 16})
    for split, hint in (("Lb0E", True), ("Lb1E", False)):
        body = kernel_body(asm, "sgemm_mfma_direct_kernel", frag + "Li2E" + split)
        stores = re.findall(r"^\s+(buffer_store\S*)\s+([^\n]*)$", body, re.M)
        got = {}
        for op, _ in stores:
            got[op] = got.get(op, 0) + 1
        assert got == want, split
        assert all(ops.rstrip().endswith(" nt") == hint for _, ops in stores), split
