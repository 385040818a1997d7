"""GPU parity of sgemm_ws, K split across workgroups, against the CPU oracle:
within 1e-5 (|A|·|B|) on random data and bit-exact on integer data, on
under-filled long-K shapes (ragged in M, N and K, rows only 4-byte aligned,
NaN padding that must not be read); the workspace is written only inside the
plan's workspace_bytes, repeated calls give the same bits, and without room
for a split the call is sgemm() bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import seedgen

from gpu_util import DevMat, assert_close, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GUARD = 1024   # floats past the workspace that must keep their sentinel
SENTINEL = np.float32(-7.25)


class Workspace:
    """A device buffer of ``nbytes`` followed by a sentinel guard region."""

    def __init__(self, nbytes: int, off: int = 0):
        assert nbytes % 4 == 0
        self.n = nbytes // 4
        self.off = off
        flat = np.full(off + self.n + GUARD, SENTINEL, np.float32)
        flat[off:off + self.n] = np.nan
        self.buf = torch.from_numpy(flat).to("cuda:0")

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + 4 * self.off

    def guards_intact(self, used_bytes: int) -> bool:
        flat = self.buf.cpu().numpy()
        before = flat[:self.off]
        after = flat[self.off + used_bytes // 4:]
        untouched = flat[self.off:self.off + self.n][used_bytes // 4:]
        return bool(np.all(before == SENTINEL) and
                    np.all(after[-GUARD:] == SENTINEL) and
                    np.all(np.isnan(untouched)))


def plan_ws(M, N, K, dA, dB, dC, nbytes):
    import tiled_fp32_gemm_amd as sg
    st, p = sg.sgemm_plan_query_ws(M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr,
                                   dC.ld, nbytes)
    assert st == sg.OK, sg.sgemm_status_string(st)
    return p


def run_ws(M, N, K, dA, dB, dC, ws: Workspace, nbytes=None):
    import tiled_fp32_gemm_amd as sg
    nbytes = ws.n * 4 if nbytes is None else nbytes
    st = sg.sgemm_ws(M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr, dC.ld,
                     torch.cuda.current_stream().cuda_stream, ws.ptr, nbytes)
    assert st == sg.OK, sg.sgemm_status_string(st)
    torch.cuda.synchronize()


def run_plain(M, N, K, dA, dB, dC):
    import tiled_fp32_gemm_amd as sg
    st = sg.sgemm(M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr, dC.ld,
                  torch.cuda.current_stream().cuda_stream)
    assert st == sg.OK, sg.sgemm_status_string(st)
    torch.cuda.synchronize()


# (M, N, K, lda, ldb, ldc, A offset in floats, distribution, seed)
SPLIT_SHAPES = [
    (256, 256, 8192, 8192, 256, 256, 0, "uniform", 1),
    (200, 300, 10001, 10003, 301, 303, 1, "normal", 2),   # ragged, 4B-aligned A
    (64, 64, 65536, 65536, 64, 64, 0, "normal", 3),
    (32, 4096, 4096, 4096, 4096, 4096, 0, "uniform", 4),
    (768, 768, 12288, 12288, 768, 768, 0, "normal", 5),
    (1000, 700, 5000, 5001, 700, 701, 0, "uniform", 6),
    (1, 1024, 65536, 65536, 1024, 1024, 0, "normal", 7),
    (1024, 1, 32768, 32768, 1, 1, 0, "normal", 8),
    (97, 131, 7777, 7779, 133, 131, 3, "uniform", 9),
    # K a multiple of 4 ending inside a slab: whole A groups of NaN padding
    # past k = K in the last split's last slab
    (256, 256, 8180, 8192, 256, 256, 0, "normal", 10),
]


def pad_inputs(M, N, K, lda, ldb, dist, seed):
    A = np.full((M, lda), np.nan, np.float32)
    B = np.full((K, ldb), np.nan, np.float32)
    a, b = seedgen.gemm_inputs(M, N, K, dist, seed)
    A[:, :K] = a
    B[:, :N] = b
    return A, B


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_split_within_tolerance(shape):
    import tiled_fp32_gemm_amd as sg
    M, N, K, lda, ldb, ldc, aoff, dist, seed = shape
    A, B = pad_inputs(M, N, K, lda, ldb, dist, seed)
    dA, dB = DevMat(A, off=aoff), DevMat(B)
    dC = DevMat(np.full((M, ldc), np.nan, np.float32))
    need = sg.sgemm_workspace_bytes(M, N, K)
    ws = Workspace(need + 64, off=1)   # 4-byte aligned only, room to spare
    p = plan_ws(M, N, K, dA, dB, dC, need + 64)
    say(f"[gpu] split {M}x{N}x{K} {p.kernel.decode()} splits={p.splits}")
    assert p.splits > 1 and p.workspace_bytes == need
    run_ws(M, N, K, dA, dB, dC, ws)
    C = dC.host()
    assert np.all(np.isnan(C[:, N:])), "C padding written"
    Cref, T = oracle.gemm(A[:, :K], B[:, :N], M=M, N=N, K=K)
    err = assert_close(C[:, :N], Cref, T, f"split {M}x{N}x{K}")
    say(f"  max normalised error {err:.3e}")
    assert ws.guards_intact(p.workspace_bytes), "workspace written out of range"


# 512 x 645 x 16384 splits with 64 x 128 tiles, whose partial tiles leave the
# kernel as column pairs: N = 645 ends five columns into the last tile.
@pytest.mark.parametrize("M,N,K", [(256, 256, 8192), (131, 97, 6001), (32, 4096, 4096),
                                   (512, 645, 16384)])
def test_split_integer_data_bitexact(M, N, K):
    import tiled_fp32_gemm_amd as sg
    A = seedgen.integer_matrix(M, K, -8, 8, 40 + K)
    B = seedgen.integer_matrix(K, N, -8, 8, 40 + K, start=M * K)
    dA, dB = DevMat(A), DevMat(B)
    dC = DevMat(np.full((M, N), np.nan, np.float32))
    need = sg.sgemm_workspace_bytes(M, N, K)
    assert need > 0
    ws = Workspace(need)
    say(f"[gpu] split int {M}x{N}x{K} ws={need}")
    run_ws(M, N, K, dA, dB, dC, ws)
    Cref, _ = oracle.gemm(A, B, M=M, N=N, K=K, with_t=False)
    assert np.array_equal(dC.host(), Cref.astype(np.float32))


def test_split_is_deterministic():
    import tiled_fp32_gemm_amd as sg
    M, N, K = 384, 384, 8192
    A, B = seedgen.gemm_inputs(M, N, K, "normal", 77)
    dA, dB = DevMat(A), DevMat(B)
    need = sg.sgemm_workspace_bytes(M, N, K)
    ws = Workspace(need)
    out = []
    for rep in range(3):
        dC = DevMat(np.full((M, N), np.nan, np.float32))
        say(f"[gpu] split determinism rep {rep}")
        run_ws(M, N, K, dA, dB, dC, ws)
        out.append(dC.host())
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])


def test_smaller_workspace_smaller_split():
    """A workspace too small for the best split takes a plan that fits it (a
    smaller split, or none: then the result is sgemm's, bit for bit)."""
    import tiled_fp32_gemm_amd as sg
    M, N, K = 256, 256, 8192
    A, B = seedgen.gemm_inputs(M, N, K, "uniform", 78)
    dA, dB = DevMat(A), DevMat(B)
    dRef = DevMat(np.full((M, N), np.nan, np.float32))
    run_plain(M, N, K, dA, dB, dRef)
    need = sg.sgemm_workspace_bytes(M, N, K)
    Cref, T = oracle.gemm(A, B)
    for nbytes in (need // 2, 3 * M * N * 4, 2 * M * N * 4, 2 * M * N * 4 - 4, 0):
        ws = Workspace(max(nbytes, 4))
        dC = DevMat(np.full((M, N), np.nan, np.float32))
        p = plan_ws(M, N, K, dA, dB, dC, nbytes)
        say(f"[gpu] split ws={nbytes}: {p.kernel.decode()} splits={p.splits}")
        assert p.workspace_bytes <= nbytes
        run_ws(M, N, K, dA, dB, dC, ws, nbytes)
        if p.splits == 1:
            assert np.array_equal(dC.host(), dRef.host())
            assert ws.guards_intact(0)
        else:
            assert_close(dC.host(), Cref, T, f"ws={nbytes}")
            assert ws.guards_intact(p.workspace_bytes)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (1000, 1500, 777), (100, 70, 0)])
def test_no_split_shapes_match_sgemm_bitwise(M, N, K):
    import tiled_fp32_gemm_amd as sg
    A, B = seedgen.gemm_inputs(M, N, max(K, 1), "uniform", 79)
    A = np.ascontiguousarray(A[:, :max(K, 1)])
    dA, dB = DevMat(A), DevMat(B)
    dRef = DevMat(np.full((M, N), np.nan, np.float32))
    dC = DevMat(np.full((M, N), np.nan, np.float32))
    ws = Workspace(1 << 20)
    say(f"[gpu] no-split {M}x{N}x{K}")
    assert sg.sgemm_workspace_bytes(M, N, K) == 0
    run_plain(M, N, K, dA, dB, dRef)
    run_ws(M, N, K, dA, dB, dC, ws)
    assert np.array_equal(dC.host(), dRef.host())
    assert ws.guards_intact(0)


def test_repeated_calls_with_a_shared_workspace():
    """Calls of different shapes on one stream reuse one workspace; each
    result stands on its own (no state carried over from the call before)."""
    import tiled_fp32_gemm_amd as sg
    ws = Workspace(64 << 20)
    for idx, (M, N, K) in enumerate([(512, 512, 16384), (64, 64, 65536), (300, 200, 30000)]):
        A, B = seedgen.gemm_inputs(M, N, K, "normal", 90 + idx)
        dA, dB = DevMat(A), DevMat(B)
        dC = DevMat(np.full((M, N), np.nan, np.float32))
        p = plan_ws(M, N, K, dA, dB, dC, ws.n * 4)
        say(f"[gpu] shared ws {M}x{N}x{K} {p.kernel.decode()}")
        assert p.splits > 1
        run_ws(M, N, K, dA, dB, dC, ws)
        Cref, T = oracle.gemm(A, B)
        assert_close(dC.host(), Cref, T, f"shared ws {M}x{N}x{K}")


def test_split_power_of_two_scaling_is_exact():
    """C(2A) = 2 C(A) and C(A/4) = C(A)/4 bit for bit through the split
    path: scaling by a power of two commutes with every rounding of both
    passes."""
    import tiled_fp32_gemm_amd as sg
    M, N, K = 256, 256, 8192
    A, B = seedgen.gemm_inputs(M, N, K, "uniform", 89)
    dB = DevMat(B)
    ws = Workspace(sg.sgemm_workspace_bytes(M, N, K))
    res = []
    for scale in (1.0, 2.0, 0.25):
        dA = DevMat((A * np.float32(scale)).astype(np.float32))
        dC = DevMat(np.full((M, N), np.nan, np.float32))
        say(f"[gpu] split scaling x{scale}")
        run_ws(M, N, K, dA, dB, dC, ws)
        res.append(dC.host())
    assert np.array_equal(res[1], 2.0 * res[0])
    assert np.array_equal(res[2], 0.25 * res[0])


def test_matmul_with_a_workspace_tensor():
    """The tensor convenience with a workspace: K split across workgroups on
    an under-filled long-K shape, within tolerance of the oracle; a bad
    workspace or algo is refused before any launch."""
    import tiled_fp32_gemm_amd as sg
    M, N, K = 200, 300, 10001
    A, B = seedgen.gemm_inputs(M, N, K, "normal", 95)
    tA, tB = torch.from_numpy(A).to("cuda:0"), torch.from_numpy(B).to("cuda:0")
    need = sg.sgemm_workspace_bytes(M, N, K)
    assert need > 0
    ws = torch.empty(need // 4, device="cuda:0")
    say(f"[gpu] matmul with workspace {M}x{N}x{K} ({need} bytes)")
    out = sg.matmul(tA, tB, workspace=ws)
    torch.cuda.synchronize()
    Cref, T = oracle.gemm(A, B)
    assert_close(out.cpu().numpy(), Cref, T, "matmul workspace")
    with pytest.raises(ValueError):
        sg.matmul(tA, tB, algo="fma", workspace=ws)
    with pytest.raises(ValueError):
        sg.matmul(tA, tB, workspace=ws.cpu())
