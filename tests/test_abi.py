"""The C-ABI library without a GPU: it loads, exports what the header
declares, and rejects bad arguments before any HIP call (CPU only)."""
from __future__ import annotations

import os
import re

import pytest

import tiled_fp32_gemm_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")

BIG = 1 << 33  # a plausible, 16-byte aligned fake device address
FAR_B, FAR_C = BIG + (1 << 40), BIG + (1 << 41)   # past any operand at BIG


@pytest.fixture(scope="module")
def lib():
    from tiled_fp32_gemm_amd import build
    build.ensure_built()
    return sg.load()


def header_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, re.M)


def test_header_declares_the_binding_names():
    assert sorted(header_functions()) == sorted(sg.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_probe_library_exports_its_header():
    # the benchmark's measurement aids: a library and header of their own
    import ctypes

    from tiled_fp32_gemm_amd import build, probe
    build.ensure_built()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "sgemm_probe.h")).read(),
                  flags=re.S)
    names = re.findall(r"^\s*int\s+(\w+)\s*\(", text, re.M)
    assert sorted(names) == ["sgemm_probe_mfma_clock", "sgemm_probe_versions"]
    plib = ctypes.CDLL(build.PROBE_LIB)
    for name in names:
        assert hasattr(plib, name), name
    # argument checks answered before any HIP call
    assert probe.mfma_clock(0, 0, 1 << 33) == 1
    assert probe.mfma_clock(0, 16, 0) == 1
    assert probe.mfma_clock(0, 16, (1 << 33) + 4) == 1


def test_one_hip_runtime_is_mapped(lib):
    maps = open("/proc/self/maps").read()
    paths = set(re.findall(r"(\S*libamdhip64\.so\S*)", maps))
    assert len(paths) == 1, paths


def test_version_and_status_strings(lib):
    assert sg.sgemm_version() == 130
    assert sg.sgemm_status_string(sg.OK) == "success"
    for st in (sg.ERR_INVALID_ARG, sg.ERR_UNSUPPORTED, sg.ERR_LAUNCH,
               sg.ERR_SCRATCH_LIMIT):
        assert sg.sgemm_status_string(st) not in ("", "success")
    assert sg.sgemm_status_string(12345) == "unknown status"


def call(M, N, K, A=BIG, lda=None, B=BIG + (1 << 31), ldb=None,
         C=BIG + (1 << 32), ldc=None, algo=0):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    st, plan = sg.sgemm_plan_query(M, N, K, A, lda, B, ldb, C, ldc, algo)
    return st, plan


@pytest.mark.parametrize("args,status", [
    (dict(M=-1, N=4, K=4), sg.ERR_INVALID_ARG),
    (dict(M=4, N=-1, K=4), sg.ERR_INVALID_ARG),
    (dict(M=4, N=4, K=-1), sg.ERR_INVALID_ARG),
    (dict(M=4, N=4, K=8, lda=7), sg.ERR_INVALID_ARG),       # lda < K
    (dict(M=4, N=8, K=4, ldb=7), sg.ERR_INVALID_ARG),       # ldb < N
    (dict(M=4, N=8, K=4, ldc=7), sg.ERR_INVALID_ARG),       # ldc < N
    (dict(M=4, N=4, K=4, lda=0), sg.ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, A=0), sg.ERR_INVALID_ARG),         # null A
    (dict(M=4, N=4, K=4, B=0), sg.ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, C=0), sg.ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, A=BIG + 2), sg.ERR_INVALID_ARG),   # not 4-byte aligned
    (dict(M=4, N=4, K=4, C=BIG + 1), sg.ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, C=BIG + 16), sg.ERR_INVALID_ARG),  # C overlaps A
    (dict(M=4, N=4, K=4, B=BIG + (1 << 32) + 60), sg.ERR_INVALID_ARG),  # B overlaps C
    (dict(M=4, N=4, K=4, algo=5), sg.ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, algo=-1), sg.ERR_INVALID_ARG),
    # operands far apart, so that only the size limits can reject
    (dict(M=(1 << 31) - 1023, N=4, K=4, B=FAR_B, C=FAR_C), sg.ERR_UNSUPPORTED),
    (dict(M=64, N=4, K=8, lda=1 << 25, B=FAR_B, C=FAR_C), sg.ERR_UNSUPPORTED),
    (dict(M=4, N=4, K=64, ldb=1 << 26, B=FAR_B, C=FAR_C), sg.ERR_UNSUPPORTED),
    (dict(M=64, N=4, K=4, ldc=1 << 26, B=FAR_B, C=FAR_C), sg.ERR_UNSUPPORTED),
    (dict(M=(1 << 29) - 1, N=1, K=1, algo=1, B=FAR_B, C=FAR_C), sg.ERR_UNSUPPORTED),
])
def test_rejected_before_any_hip_call(lib, args, status):
    st, _ = call(**args)
    assert st == status
    # the launching entry points apply the same checks and launch nothing
    M, N, K = args["M"], args["N"], args["K"]
    a = dict(A=BIG, B=BIG + (1 << 31), C=BIG + (1 << 32))
    a.update({k: v for k, v in args.items() if k in ("A", "B", "C")})
    lda = args.get("lda", max(K, 1))
    ldb = args.get("ldb", max(N, 1))
    ldc = args.get("ldc", max(N, 1))
    assert sg.sgemm_ex(M, N, K, a["A"], lda, a["B"], ldb, a["C"], ldc, 0,
                       args.get("algo", 0)) == status
    if "algo" not in args:
        assert sg.sgemm(M, N, K, a["A"], lda, a["B"], ldb, a["C"], ldc, 0) == status


def test_empty_problems_are_noops(lib):
    # nothing is touched when M or N is 0, so the pointers may be null
    assert sg.sgemm(0, 5, 5, 0, 5, 0, 5, 0, 5, 0) == sg.OK
    assert sg.sgemm(5, 0, 5, 0, 5, 0, 1, 0, 1, 0) == sg.OK
    st, plan = call(0, 8, 8)
    assert st == sg.OK and plan.workgroups == 0


@pytest.mark.parametrize("algo", sorted(sg.ALGOS))
def test_k_zero_plans_a_zero_fill(lib, algo):
    # neither A nor B is read, so null, unaligned or narrow ones are fine
    for a, lda in ((0, 1), (BIG + 4, 3)):
        st, plan = call(100, 70, 0, A=a, lda=lda, B=0, algo=sg.ALGOS[algo])
        assert st == sg.OK and plan.workgroups > 0 and plan.kernel


@pytest.mark.parametrize("M,N,K,lda,ldb,aoff,kernel,wgs", [
    (4096, 4096, 4096, 4096, 4096, 0, "mfma_lds_256x256x32_vavb", 256),
    (8192, 8192, 8192, 8192, 8192, 0, "mfma_lds_256x256x32_vavb", 1024),
    (65536, 128, 256, 256, 128, 0, "mfma_lds_128x128x32_vavb", 512),
    (1000, 1500, 777, 777, 1500, 0, "mfma_lds_32x64x32_ks2_savb", 768),
    (256, 256, 256, 256, 256, 0, "mfma_lds_32x64x64_ks4_vavb", 32),
    (256, 256, 256, 256, 256, 4, "mfma_lds_32x64x64_ks4_savb", 32),  # A 4B-aligned
    (256, 256, 256, 258, 256, 0, "mfma_lds_32x64x64_ks4_savb", 32),  # lda % 4 != 0
    (4096, 4096, 4095, 4095, 4096, 0, "mfma_lds_256x256x32_savb", 256),
    (3000, 3000, 512, 512, 3000, 0, "mfma_lds_64x64x32_vavb", 2209),
    (2048, 2048, 2048, 2048, 2048, 0, "mfma_lds_64x128x32_vavb", 512),
    (512, 4096, 4096, 4096, 4096, 0, "mfma_lds_64x64x32_vavb", 512),
    (384, 4096, 64, 64, 4096, 0, "mfma_lds_32x64x32_ks2_vavb", 768),
])
def test_plans(lib, M, N, K, lda, ldb, aoff, kernel, wgs):
    st, plan = call(M, N, K, A=BIG + aoff, lda=lda, ldb=ldb,
                    B=BIG + (1 << 31), C=BIG + (1 << 32))
    assert st == sg.OK
    assert plan.kernel.decode() == kernel and plan.workgroups == wgs
    assert plan.algo == sg.ALGOS["mfma_direct"]


def test_register_staged_family_plans(lib):
    st, plan = call(1000, 1500, 777, lda=777, algo=sg.ALGOS["mfma"])
    assert st == sg.OK and plan.kernel.decode() == "mfma_64x64x16_savb"
    st, plan = call(4096, 4096, 4096, algo=sg.ALGOS["mfma"])
    assert st == sg.OK and plan.kernel.decode() == "mfma_256x128x16_vavb"


def test_plans_per_family(lib):
    for name, prefix in (("simple", "simple_"), ("fma", "fma_"), ("mfma", "mfma_"),
                         ("mfma_direct", "mfma_lds_")):
        st, plan = call(300, 200, 100, lda=100, algo=sg.ALGOS[name])
        assert st == sg.OK and plan.kernel.decode().startswith(prefix)
        assert plan.lds_bytes <= 160 * 1024


@pytest.mark.parametrize("args,status", [
    (dict(rows=-1, cols=4), sg.ERR_INVALID_ARG),
    (dict(rows=4, cols=8, ldi=7), sg.ERR_INVALID_ARG),       # ldi < cols
    (dict(rows=8, cols=4, ldo=7), sg.ERR_INVALID_ARG),       # ldo < rows
    (dict(rows=4, cols=4, inp=0), sg.ERR_INVALID_ARG),
    (dict(rows=4, cols=4, out=BIG + 2), sg.ERR_INVALID_ARG),
    (dict(rows=4, cols=4, out=BIG + 32), sg.ERR_INVALID_ARG),  # overlap
    (dict(rows=4, cols=4, layout=4), sg.ERR_INVALID_ARG),
    # one tile's input rows (64) or output rows (128) spanning 2 GiB or
    # more, a dimension past the limit, a grid of 2^32 work-items
    (dict(rows=64, cols=4, ldi=1 << 25, out=FAR_C), sg.ERR_UNSUPPORTED),
    (dict(rows=4, cols=128, ldo=1 << 25, out=FAR_C), sg.ERR_UNSUPPORTED),
    (dict(rows=(1 << 31) - 1023, cols=1, out=FAR_C), sg.ERR_UNSUPPORTED),
    (dict(rows=(1 << 31) - 1024, cols=1, out=FAR_C), sg.ERR_UNSUPPORTED),
    (dict(rows=0, cols=4, inp=0, out=0), sg.OK),
])
def test_transpose_checks(lib, args, status):
    rows, cols = args["rows"], args["cols"]
    inp = args.get("inp", BIG)
    out = args.get("out", BIG + (1 << 32))
    ldi = args.get("ldi", max(cols, 1))
    ldo = args.get("ldo", max(rows, 1))
    assert sg.sgemm_transpose_ex(rows, cols, inp, ldi, out, ldo, 0,
                                 args.get("layout", 0)) == status


def test_ladder_steps_and_names(lib):
    names = sg.ladder_steps()
    assert len(names) == sg.sgemm_ladder_steps() == 14
    assert names[0] == "naive_global" and names[-1] == "mfma_direct_to_lds"
    assert sg.sgemm_ladder_name(-1) is None and sg.sgemm_ladder_name(14) is None


@pytest.mark.parametrize("step", [0, 5, 9, 11, 13])
def test_ladder_checks_before_any_hip_call(lib, step):
    # the same checks as sgemm, all answered on the host
    B, C = BIG + (1 << 31), BIG + (1 << 32)
    assert sg.sgemm_ladder(step, -1, 4, 4, BIG, 4, B, 4, C, 4) == sg.ERR_INVALID_ARG
    assert sg.sgemm_ladder(step, 4, 4, 8, BIG, 7, B, 4, C, 4) == sg.ERR_INVALID_ARG   # lda < K
    assert sg.sgemm_ladder(step, 4, 4, 4, BIG, 4, B, 4, BIG + 8, 4) == sg.ERR_INVALID_ARG  # overlap
    assert sg.sgemm_ladder(step, 4, 4, 4, 0, 4, B, 4, C, 4) == sg.ERR_INVALID_ARG
    assert sg.sgemm_ladder(step, 0, 5, 5, 0, 5, 0, 5, 0, 5) == sg.OK   # nothing to do


def test_ladder_rejects_unknown_steps(lib):
    B, C = BIG + (1 << 31), BIG + (1 << 32)
    for step in (-1, 14, 1 << 20):
        assert sg.sgemm_ladder(step, 4, 4, 4, BIG, 4, B, 4, C, 4) == sg.ERR_INVALID_ARG


# Split K across workgroups (sgemm_ws): plans, sizes and argument checks.
WS = BIG + (3 << 31)   # a fake workspace address past A, B and C


def call_ws(M, N, K, ws_bytes, lda=None, ldb=None, ldc=None):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return sg.sgemm_plan_query_ws(M, N, K, BIG, lda, BIG + (1 << 31), ldb,
                                  BIG + (1 << 32), ldc, ws_bytes)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (256, 256, 8192),
                                   (1000, 1500, 777), (64, 64, 65536),
                                   (100, 70, 0), (0, 8, 8)])
def test_ws_plan_without_workspace_is_the_plain_plan(lib, M, N, K):
    st0, p0 = call(M, N, K)
    st1, p1 = call_ws(M, N, K, 0)
    assert st0 == st1 == sg.OK
    assert p1.as_dict() == p0.as_dict()
    assert p1.splits == 1 and p1.workspace_bytes == 0


@pytest.mark.parametrize("M,N,K", [(256, 256, 8192), (64, 64, 65536),
                                   (32, 4096, 4096), (200, 300, 10001),
                                   (768, 768, 12288), (1, 1024, 65536),
                                   (1024, 1, 32768)])
def test_split_plans_for_underfilled_long_k(lib, M, N, K):
    need = sg.sgemm_workspace_bytes(M, N, K)
    st, p = call_ws(M, N, K, need)
    assert st == sg.OK and need > 0
    assert p.splits > 1 and p.workspace_bytes == need == p.splits * M * N * 4
    assert p.kernel.decode().endswith(f"_split{p.splits}")
    assert p.workgroups == -(-M // p.tile_m) * -(-N // p.tile_n) * p.splits
    # a larger workspace gives the same plan; a smaller one a smaller split
    # that fits it, or none
    assert call_ws(M, N, K, 1 << 30)[1].as_dict() == p.as_dict()
    st2, p2 = call_ws(M, N, K, need - 4)
    assert st2 == sg.OK and p2.workspace_bytes <= need - 4
    assert p2.splits < p.splits or p2.as_dict() != p.as_dict()
    st3, p3 = call_ws(M, N, K, 2 * M * N * 4 - 4)   # not even two partials
    assert st3 == sg.OK and p3.splits == 1 and p3.workspace_bytes == 0


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (8192, 8192, 8192),
                                   (65536, 128, 256), (256, 256, 256),
                                   (2048, 2048, 2048), (100, 100, 0)])
def test_no_split_where_the_chip_is_filled(lib, M, N, K):
    assert sg.sgemm_workspace_bytes(M, N, K) == 0
    st, p = call_ws(M, N, K, 1 << 30)
    assert st == sg.OK and p.splits == 1 and p.as_dict() == call(M, N, K)[1].as_dict()


def test_workspace_bytes_of_invalid_or_empty_shapes(lib):
    for M, N, K in ((-1, 4, 4), (4, -1, 4), (4, 4, -1), (0, 4, 4096), (4, 0, 4096)):
        assert sg.sgemm_workspace_bytes(M, N, K) == 0


def test_ws_argument_checks_before_any_hip_call(lib):
    M, N, K = 256, 256, 8192
    need = sg.sgemm_workspace_bytes(M, N, K)
    A, B, C = BIG, BIG + (1 << 31), BIG + (1 << 32)
    bad = [(WS, -4), (0, need), (WS + 2, need),      # negative, null, misaligned
           (A + 64, need), (B, need), (C - 16, need)]  # overlaps A, B, C
    for ws, nb in bad:
        assert sg.sgemm_ws(M, N, K, A, K, B, N, C, N, 0, ws, nb) == sg.ERR_INVALID_ARG, (ws, nb)
    # the sgemm checks come first, and apply with a workspace as well
    assert sg.sgemm_ws(M, N, K, A, K - 1, B, N, C, N, 0, WS, need) == sg.ERR_INVALID_ARG
    assert sg.sgemm_ws(M, N, K, 0, K, B, N, C, N, 0, WS, need) == sg.ERR_INVALID_ARG
    assert sg.sgemm_ws(0, N, K, 0, K, 0, N, 0, N, 0, 0, 0) == sg.OK   # empty: no-op
    st, _ = sg.sgemm_plan_query_ws(M, N, K, A, K, B, N, C, N, -1)
    assert st == sg.ERR_INVALID_ARG
    assert lib.sgemm_plan_query_ws(M, N, K, A, K, B, N, C, N, need, None) == sg.ERR_INVALID_ARG
