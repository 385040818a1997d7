"""Size limits of the C ABI.

The kernels address each operand from the corner of their own C tile (A from
the tile's first row, B from a slab's first row and the tile's first column,
C from the tile's corner) with 32-bit byte offsets, so an operand may be of
any size; what is bounded is one tile's span (2 GiB), each dimension (below
2^31 - 1024) and the grid (below 2^32 work-items).  The CPU tests check the
plans and rejections through ``sgemm_plan_query`` (no HIP call); the GPU
tests run every kernel family on operands of 3 GiB against the oracle on
sampled rows or columns, bit-exact on integer data, where every kernel
offset is formed from the tile's corner ("CUDA in depth (5): vectorized load
and shared-memory layout", sections on leading dimensions and on edges).
"""
from __future__ import annotations

import numpy as np
import pytest

import tiled_fp32_gemm_amd as sg

BIG = 1 << 33                      # fake, 16-byte aligned device addresses,
FAR_B, FAR_C = BIG + (1 << 40), BIG + (1 << 41)   # far enough apart
GIB = 1 << 30
FAMILIES = ["auto", "mfma_direct", "mfma", "fma", "simple"]


@pytest.fixture(scope="module")
def lib():
    from tiled_fp32_gemm_amd import build
    build.ensure_built()
    return sg.load()


def plan(M, N, K, lda=None, ldb=None, ldc=None, algo="auto", aoff=0):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return sg.sgemm_plan_query(M, N, K, BIG + aoff, lda, FAR_B, ldb, FAR_C, ldc,
                               sg.ALGOS[algo])


# -- CPU: plans and rejections ----------------------------------------------

# (M, N, K): A, B or C of 3 GiB and of 5 GiB, with 16-byte-aligned rows.
BIG_SHAPES = [(49152, 64, 16384), (81920, 64, 16384),     # A
              (32, 65536, 12288), (32, 65536, 20480),     # B
              (65536, 12288, 4), (65536, 20480, 4)]       # C


@pytest.mark.parametrize("algo", FAMILIES)
@pytest.mark.parametrize("M,N,K", BIG_SHAPES)
def test_operands_past_2_and_4_gib_are_planned(lib, algo, M, N, K):
    st, p = plan(M, N, K, algo=algo)
    assert st == sg.OK, sg.sgemm_status_string(st)
    assert p.workgroups == -(-M // p.tile_m) * -(-N // p.tile_n)


def test_unaligned_rows_past_2_gib_are_planned(lib):
    for algo in FAMILIES:
        st, p = plan(49155, 64, 16383, algo=algo, aoff=4)
        assert st == sg.OK and not p.vec_a


def test_the_planner_keeps_to_tiles_whose_span_fits(lib):
    # 16 MiB rows of A: a 256-row tile spans 4 GiB, a 128-row one just under 2
    st, p = plan(4096, 4096, 32, lda=1 << 22)
    assert st == sg.OK and p.tile_m <= 128
    # 32 MiB rows: only tiles of 64 rows or fewer
    st, p = plan(4096, 4096, 32, lda=1 << 23)
    assert st == sg.OK and p.tile_m <= 64
    # 128 MiB rows: even 32 rows span 4 GiB
    assert plan(4096, 4096, 32, lda=1 << 25)[0] == sg.ERR_UNSUPPORTED
    # the same for C's rows, and for a slab's rows of B
    st, p = plan(4096, 4096, 32, ldc=1 << 23)
    assert st == sg.OK and p.tile_m <= 64
    assert plan(4096, 64, 4096, ldb=1 << 26)[0] == sg.ERR_UNSUPPORTED


def test_two_rows_with_a_huge_pitch(lib):
    # two rows of A 1 GiB apart: any tile covers both, 1 GiB + 32 floats
    for algo in FAMILIES:
        assert plan(2, 64, 8, lda=1 << 28, algo=algo)[0] == sg.OK
    # 2 GiB apart: no tile can reach the second row
    assert plan(2, 64, 8, lda=1 << 29)[0] == sg.ERR_UNSUPPORTED
    # a single row never uses its pitch
    assert plan(1, 64, 8, lda=1 << 40)[0] == sg.OK


def test_dimension_limit(lib):
    lim = (1 << 31) - 1024
    assert plan(lim + 1, 1, 1)[0] == sg.ERR_UNSUPPORTED
    assert plan(1, lim + 1, 1)[0] == sg.ERR_UNSUPPORTED
    assert plan(1, 1, lim + 1)[0] == sg.ERR_UNSUPPORTED
    # at the limit the other rules decide: M = lim makes no grid below 2^32
    # work-items, and K = lim puts 8 GiB in one row of A; a row of A just
    # under 2 GiB is fine
    assert plan(lim, 1, 1)[0] == sg.ERR_UNSUPPORTED
    assert plan(1, 1, lim)[0] == sg.ERR_UNSUPPORTED
    assert plan(1, 1, (1 << 29) - 64)[0] == sg.OK


def test_grid_limit(lib):
    # 16 x 16 tiles of 256 threads: 2^25 of them are 2^33 work-items
    M = (1 << 29) - 1
    assert plan(M, 1, 1, algo="simple")[0] == sg.ERR_UNSUPPORTED
    assert sg.sgemm_ex(M, 1, 1, BIG, 1, FAR_B, 1, FAR_C, 1, 0,
                       sg.ALGOS["simple"]) == sg.ERR_UNSUPPORTED
    for step in (0, 1, 2):   # the ladder's 16 x 16 tile steps
        assert sg.sgemm_ladder(step, M, 1, 1, BIG, 1, FAR_B, 1, FAR_C, 1, 0) \
            == sg.ERR_UNSUPPORTED
    st, p = plan(M, 1, 1)     # larger tiles keep the grid small
    assert st == sg.OK and p.workgroups * p.threads < (1 << 32)


def test_short_k_with_a_huge_ldb_is_planned(lib):
    # slab rows past K would sit 2^31 bytes or more away; they read zeros
    st, p = plan(4096, 64, 2, ldb=40_000_003)
    assert st == sg.OK and p.algo == sg.ALGOS["mfma_direct"]
    # up to 14 rows of B fit in 2 GiB at that pitch; 15 or more do not
    assert plan(4096, 64, 14, ldb=40_000_003)[0] == sg.OK
    assert plan(4096, 64, 15, ldb=40_000_003)[0] == sg.ERR_UNSUPPORTED


def test_split_workspace_stays_below_2_gib(lib):
    for M, N, K in ((256, 256, 3 << 20), (1024, 1024, 1 << 20), (64, 64, 1 << 22)):
        need = sg.sgemm_workspace_bytes(M, N, K)
        assert 0 < need < 2 * GIB


# -- GPU: every family on 3 GiB operands ---------------------------------------

def _int_matrix(rows, cols, a, b, m):
    """((a i + b j) mod m) - m // 2 as float32 on the GPU (exact integers)."""
    import torch
    i = torch.arange(rows, device="cuda:0", dtype=torch.int32)[:, None]
    j = torch.arange(cols, device="cuda:0", dtype=torch.int32)[None, :]
    return ((i * a + j * b) % m - m // 2).to(torch.float32)


def _run(M, N, K, A, lda, B, ldb, C, ldc, algo):
    import torch
    st = sg.sgemm_ex(M, N, K, A, lda, B, ldb, C, ldc,
                     torch.cuda.current_stream().cuda_stream, sg.ALGOS[algo])
    assert st == sg.OK, sg.sgemm_status_string(st)
    torch.cuda.synchronize()


def _say(*a):
    print(*a, flush=True)


@pytest.mark.gpu
@pytest.mark.parametrize("algo", ["auto", "mfma", "fma", "simple"])
@pytest.mark.parametrize("aligned", [True, False])
def test_gpu_a_of_3_gib(algo, aligned):
    import oracle
    import torch
    M, N, K = (49152, 64, 16384) if aligned else (49155, 64, 16383)
    _say(f"[gpu] A {M}x{K} ({4 * M * K / GIB:.3f} GiB) algo={algo} aligned={aligned}")
    dA = _int_matrix(M, K, 7, 3, 17)
    B = (np.arange(K * N, dtype=np.int64).reshape(K, N) * 5 % 13 - 6).astype(np.float32)
    dB = torch.from_numpy(B).to("cuda:0")
    dC = torch.full((M, N), float("nan"), device="cuda:0")
    _run(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, algo)
    rows = torch.tensor([0, 1, 4095, 4096, 20000, 32767, 32768, M - 2, M - 1],
                        device="cuda:0")
    Cref, _ = oracle.gemm(dA[rows].cpu().numpy(), B, with_t=False)
    assert np.array_equal(dC[rows].cpu().numpy(), Cref.astype(np.float32))
    assert bool(torch.isfinite(dC).all())


@pytest.mark.gpu
@pytest.mark.parametrize("algo", ["auto", "mfma", "fma", "simple"])
def test_gpu_b_of_3_gib(algo):
    import oracle
    import torch
    M, N, K = 32, 65536, 12288
    _say(f"[gpu] B {K}x{N} ({4 * K * N / GIB:.3f} GiB) algo={algo}")
    A = (np.arange(M * K, dtype=np.int64).reshape(M, K) * 3 % 11 - 5).astype(np.float32)
    dA = torch.from_numpy(A).to("cuda:0")
    dB = _int_matrix(K, N, 5, 7, 13)
    dC = torch.full((M, N), float("nan"), device="cuda:0")
    _run(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, algo)
    cols = torch.tensor([0, 1, 255, 256, 30000, 32767, 32768, N - 2, N - 1],
                        device="cuda:0")
    Bc = np.ascontiguousarray(dB[:, cols].cpu().numpy())
    Cref, _ = oracle.gemm(A, Bc, with_t=False)
    assert np.array_equal(dC[:, cols].cpu().numpy(), Cref.astype(np.float32))
    assert bool(torch.isfinite(dC).all())


@pytest.mark.gpu
@pytest.mark.parametrize("algo", ["auto", "mfma", "fma", "simple"])
def test_gpu_c_of_3_gib(algo):
    import oracle
    import torch
    M, N, K = 65536, 12288, 4
    _say(f"[gpu] C {M}x{N} ({4 * M * N / GIB:.3f} GiB) algo={algo}")
    A = (np.arange(M * K, dtype=np.int64).reshape(M, K) % 9 - 4).astype(np.float32)
    B = (np.arange(K * N, dtype=np.int64).reshape(K, N) % 7 - 3).astype(np.float32)
    dA, dB = torch.from_numpy(A).to("cuda:0"), torch.from_numpy(B).to("cuda:0")
    dC = torch.full((M, N), float("nan"), device="cuda:0")
    _run(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, algo)
    rows = np.array([0, 1, 4095, 4096, 40000, M - 2, M - 1])
    Cref, _ = oracle.gemm(A[rows], B, with_t=False)
    got = dC[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
    assert np.array_equal(got, Cref.astype(np.float32))
    assert bool(torch.isfinite(dC).all())


@pytest.mark.gpu
def test_gpu_ladder_on_a_c_of_3_gib():
    import oracle
    import torch
    M, N, K = 65536, 12288, 4
    A = (np.arange(M * K, dtype=np.int64).reshape(M, K) % 9 - 4).astype(np.float32)
    B = (np.arange(K * N, dtype=np.int64).reshape(K, N) % 7 - 3).astype(np.float32)
    dA, dB = torch.from_numpy(A).to("cuda:0"), torch.from_numpy(B).to("cuda:0")
    dC = torch.empty((M, N), device="cuda:0")
    rows = np.array([0, 1, 40000, M - 1])
    Cref = oracle.gemm(A[rows], B, with_t=False)[0].astype(np.float32)
    for step in range(sg.sgemm_ladder_steps()):
        _say(f"[gpu] ladder step {step} ({sg.sgemm_ladder_name(step)}) on a 3 GiB C")
        dC.fill_(float("nan"))
        st = sg.sgemm_ladder(step, M, N, K, dA.data_ptr(), K, dB.data_ptr(), N,
                             dC.data_ptr(), N, torch.cuda.current_stream().cuda_stream)
        assert st == sg.OK
        torch.cuda.synchronize()
        got = dC[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
        assert np.array_equal(got, Cref), step
        assert bool(torch.isfinite(dC).all()), step


@pytest.mark.gpu
def test_gpu_split_k_with_a_b_of_3_gib():
    import oracle
    import torch
    M, N, K = 256, 256, 3 << 20
    _say(f"[gpu] sgemm_ws with B {K}x{N} ({4 * K * N / GIB:.3f} GiB)")
    # A in {0, 1}, B in {-1, 0, 1}: every partial sum is an integer below 2^24
    dA = (_int_matrix(M, K, 1, 1, 2) + 1)
    dB = _int_matrix(K, N, 3, 1, 3)
    dC = torch.full((M, N), float("nan"), device="cuda:0")
    need = sg.sgemm_workspace_bytes(M, N, K)
    ws = torch.empty(need // 4, device="cuda:0")
    st, p = sg.sgemm_plan_query_ws(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N,
                                   dC.data_ptr(), N, need)
    assert st == sg.OK and p.splits > 1
    st = sg.sgemm_ws(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
                     torch.cuda.current_stream().cuda_stream, ws.data_ptr(), need)
    assert st == sg.OK
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 127, 128, 254, 255], device="cuda:0")
    cols = torch.tensor([0, 3, 64, 200, 255], device="cuda:0")
    Ar = dA[rows].cpu().numpy()
    Bc = np.ascontiguousarray(dB[:, cols].cpu().numpy())
    Cref, _ = oracle.gemm(Ar, Bc, with_t=False)
    got = dC[rows][:, cols].cpu().numpy()
    assert np.array_equal(got, Cref.astype(np.float32))
    assert bool(torch.isfinite(dC).all())


@pytest.mark.gpu
def test_gpu_transpose_of_3_gib():
    import torch
    rows, cols = 49152, 16384
    _say(f"[gpu] transpose {rows}x{cols} ({4 * rows * cols / GIB:.3f} GiB)")
    dI = _int_matrix(rows, cols, 7, 3, 1021)
    dO = torch.full((cols, rows), float("nan"), device="cuda:0")
    st = sg.sgemm_transpose(rows, cols, dI.data_ptr(), cols, dO.data_ptr(), rows,
                            torch.cuda.current_stream().cuda_stream)
    assert st == sg.OK
    torch.cuda.synchronize()
    for j in (0, 1, 127, 128, 8191, cols - 1):      # output rows = input columns
        got = dO[j].cpu().numpy()
        assert np.array_equal(got, dI[:, j].cpu().numpy()), j
    for i in (0, 63, 64, 30000, rows - 1):          # output columns = input rows
        assert np.array_equal(dO[:, i].cpu().numpy(), dI[i].cpu().numpy()), i


@pytest.mark.gpu
@pytest.mark.parametrize("K", [1, 2, 5, 14])
@pytest.mark.parametrize("algo", ["auto", "mfma"])
def test_gpu_short_k_with_huge_ldb(K, algo):
    """B rows are 40,000,003 floats apart, so the slab rows past K sit up to
    5 GB from the slab's first row (past 2^31 bytes from row 14 on); they
    must read zeros (the pages' edge rule), not wrap onto B's NaN-filled gap
    columns."""
    import oracle
    import torch
    M, N, ldb = 4096, 64, 40_000_003
    _say(f"[gpu] K={K} ldb={ldb} algo={algo}")
    A = (np.arange(M * K, dtype=np.int64).reshape(M, K) % 9 - 4).astype(np.float32)
    B = (np.arange(K * N, dtype=np.int64).reshape(K, N) % 7 - 3).astype(np.float32)
    dA = torch.from_numpy(A).to("cuda:0")
    dBbuf = torch.full(((K - 1) * ldb + N + 64,), float("nan"), device="cuda:0")
    for k in range(K):
        dBbuf[k * ldb:k * ldb + N] = torch.from_numpy(B[k]).to("cuda:0")
    dC = torch.full((M, N), float("nan"), device="cuda:0")
    _run(M, N, K, dA.data_ptr(), K, dBbuf.data_ptr(), ldb, dC.data_ptr(), N, algo)
    Cref, _ = oracle.gemm(A, B, with_t=False)
    assert np.array_equal(dC.cpu().numpy(), Cref.astype(np.float32))
