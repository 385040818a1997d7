"""Planner inputs against the built kernels (CPU only).

``sgemm_plan_query`` reports ``wg_per_cu``, the workgroups of the chosen
kernel that the planner assumes one CU holds at once, and ``lds_bytes``.  On
gfx950 the first follows from the code object: a SIMD lane has 512 registers
(VGPRs and AGPRs together, allocated in blocks of 8) and runs at most 8
waves, and a CU has 4 SIMDs and 160 KiB of LDS.  This test derives both from
the metadata of each kernel in the library's gfx950 assembly and checks the
plans of a grid of shapes, in every kernel family, against them.  A compiler
that allocates registers differently makes it fail, and the planner's table
must then be updated.
"""
from __future__ import annotations

import itertools
import re
import shutil

import pytest

import tiled_fp32_gemm_amd as sg

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None,
                                reason="needs hipcc to build the assembly")

BIG = 1 << 40
DIMS = [64, 96, 128, 256, 384, 512, 1000, 1024, 2048, 3000, 4096, 8192, 16384]
KS = [32, 128, 777, 2048, 8192]


@pytest.fixture(scope="module")
def kernels():
    """symbol -> (template ints, registers per lane, LDS bytes, max threads)."""
    from tiled_fp32_gemm_amd import build
    asm = open(build.build_asm()).read()
    meta = asm[asm.index("amdhsa.kernels:"):]
    out = {}
    for entry in re.split(r"\n  - ", meta):
        m = re.search(r"\.name:\s+(_ZN2sg\w+)", entry)
        if not m:
            continue
        get = lambda key: int(re.search(r"\." + key + r":\s+(\d+)", entry).group(1))
        args = tuple(int(x) for x in re.findall(r"Li(\d+)E", m.group(1)))
        out[m.group(1)] = (args, get("vgpr_count"),
                           get("group_segment_fixed_size"),
                           get("max_flat_workgroup_size"))
    assert out, "no kernel metadata in the assembly"
    return out


def resident(regs: int, lds: int, threads: int) -> int:
    waves_per_simd = min(8, 512 // ((regs + 7) // 8 * 8))
    by_waves = 4 * waves_per_simd // (threads // 64)
    by_lds = (160 * 1024) // lds if lds else by_waves
    return min(by_waves, by_lds)


def matching(kernels, plan):
    """The code objects the plan may launch (every load form of its tile)."""
    name = plan.kernel.decode()
    if name.startswith("mfma_lds_"):
        ks = int(re.search(r"_ks(\d+)", name).group(1)) if "_ks" in name else 1
        stages = int(re.search(r"_s(\d+)", name).group(1)) if re.search(r"_s\d", name) else 2
        want = lambda s, a: ("direct_kernel" in s and a[0] == plan.tile_m and
                             a[1] == plan.tile_n and a[4] == plan.tile_k and a[5] == ks and
                             a[6] == stages)
    elif name.startswith("mfma_"):
        want = lambda s, a: ("17sgemm_mfma_kernel" in s and a[0] == plan.tile_m and
                             a[1] == plan.tile_n and a[4] == plan.tile_k)
    elif name.startswith("fma_"):
        want = lambda s, a: "sgemm_fma_kernel" in s
    else:
        want = lambda s, a: "sgemm_simple_kernel" in s
    found = [v for s, v in kernels.items() if want(s, v[0])]
    assert found, name
    return found


@pytest.mark.parametrize("algo", ["mfma_direct", "mfma", "fma", "simple"])
def test_plans_match_the_code_objects(kernels, algo):
    seen = set()
    for M, N, K in itertools.product(DIMS, DIMS, KS):
        st, plan = sg.sgemm_plan_query(M, N, K, BIG, K, BIG + (1 << 34), N,
                                       BIG + (1 << 36), N, sg.ALGOS[algo])
        assert st == sg.OK
        name = plan.kernel.decode()[:-5]
        if name in seen:
            continue
        seen.add(name)
        for _, regs, lds, threads in matching(kernels, plan):
            assert threads == plan.threads, name
            assert lds == plan.lds_bytes, name
            assert resident(regs, lds, threads) == plan.wg_per_cu, (name, regs, lds)
    if algo == "mfma_direct":   # every LDS-direct tile is chosen somewhere
        assert len(seen) == 8, sorted(seen)
