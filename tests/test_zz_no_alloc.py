"""sgemm_ws_noalloc: sgemm_ws for callers that cannot allocate, with the
split partials in the library's static per-device scratch.

Checked through the C ABI against sgemm_ws (a caller's workspace of the same
size): the same plan and kernels, so the same bits, on two calls in a row,
the second smaller than the first; and, like every product test, against
the oracle within 1e-5 * (|A|.|B|) on sampled rows.  The first call of the
first pair goes to sgemm_ws_noalloc, so that in a fresh process it is the
call that looks the scratch up.
"""
from __future__ import annotations

import numpy as np
import pytest

import seedgen
import tiled_fp32_gemm_amd as sg

BIG = 1 << 33


def test_rejects_a_request_beyond_the_scratch_before_any_hip_call():
    M, N, K = 256, 256, 8192
    args = (M, N, K, BIG, K, BIG + (1 << 36), N, BIG + (1 << 37), N, 0)
    assert sg.sgemm_ws_noalloc(*args, sg.NOALLOC_MAX_BYTES + 4) == sg.ERR_SCRATCH_LIMIT
    assert sg.sgemm_ws_noalloc(*args, -4) == sg.ERR_INVALID_ARG
    assert "scratch" in sg.sgemm_status_string(sg.ERR_SCRATCH_LIMIT)
    # the sgemm checks apply as well, before any HIP call
    assert sg.sgemm_ws_noalloc(M, N, K, BIG, K - 1, BIG + (1 << 36), N,
                               BIG + (1 << 37), N, 0, 1 << 20) == sg.ERR_INVALID_ARG
    assert sg.sgemm_ws_noalloc(0, N, K, 0, K, 0, N, 0, N, 0, 0) == sg.OK


@pytest.mark.gpu
def test_no_alloc_matches_sgemm_ws_on_two_calls():
    import torch

    import oracle
    from gpu_util import assert_close, say
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    # the second shape is smaller than the first, in M, N, K and in scratch
    for i, (M, N, K, seed) in enumerate([(512, 512, 16384, 71), (256, 256, 8192, 72)]):
        say(f"[gpu] sgemm_ws_noalloc M={M} N={N} K={K} seed={seed}")
        A, B = seedgen.gemm_inputs(M, N, K, "uniform", seed)
        tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        need = sg.sgemm_workspace_bytes(M, N, K)
        assert 0 < need <= sg.NOALLOC_MAX_BYTES
        st, plan = sg.sgemm_plan_query_ws(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N,
                                          tB.data_ptr() + (1 << 40), N, need)
        assert st == sg.OK and plan.splits > 1
        ws = torch.empty(need // 4, dtype=torch.float32, device=dev)
        c_ws = torch.full((M, N), float("nan"), device=dev)
        c_na = torch.full((M, N), float("nan"), device=dev)

        def no_alloc():
            return sg.sgemm_ws_noalloc(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N,
                                       c_na.data_ptr(), N, stream, need)

        def with_ws():
            return sg.sgemm_ws(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N,
                               c_ws.data_ptr(), N, stream, ws.data_ptr(), need)

        order = (no_alloc, with_ws) if i == 0 else (with_ws, no_alloc)
        for call in order:
            assert call() == sg.OK
        torch.cuda.synchronize()
        got = c_na.cpu().numpy()
        assert np.array_equal(got, c_ws.cpu().numpy())
        rows = np.unique(np.array([0, 1, M // 2, M - 2, M - 1]))
        Cref, T = oracle.gemm(A[rows], B)
        err = assert_close(got[rows], Cref, T, f"sgemm_ws_noalloc {M}x{N}x{K}")
        say(f"  bit-equal to sgemm_ws; max normalised error {err:.2e}")
        del ws


@pytest.mark.gpu
def test_no_alloc_replays_under_graph_capture():
    """Captured in a HIP graph after one eager call (which makes the scratch
    lookup), the split product replays to the eager bits; eager calls of
    another shape between the replays overwrite the shared scratch, which
    each replay rewrites before it reads."""
    import torch

    from gpu_util import say
    dev = torch.device("cuda:0")
    M, N, K = 256, 256, 8192
    A, B = seedgen.gemm_inputs(M, N, K, "uniform", 73)
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    need = sg.sgemm_workspace_bytes(M, N, K)
    assert 0 < need <= sg.NOALLOC_MAX_BYTES
    C = torch.empty((M, N), device=dev)
    M2, N2, K2 = 200, 300, 10001
    A2, B2 = seedgen.gemm_inputs(M2, N2, K2, "uniform", 74)
    tA2, tB2 = torch.from_numpy(A2).to(dev), torch.from_numpy(B2).to(dev)
    need2 = sg.sgemm_workspace_bytes(M2, N2, K2)
    assert 0 < need2 <= sg.NOALLOC_MAX_BYTES
    C2 = torch.empty((M2, N2), device=dev)

    def call():
        s = torch.cuda.current_stream().cuda_stream
        return sg.sgemm_ws_noalloc(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N,
                                   C.data_ptr(), N, s, need)

    def other():
        s = torch.cuda.current_stream().cuda_stream
        return sg.sgemm_ws_noalloc(M2, N2, K2, tA2.data_ptr(), K2, tB2.data_ptr(), N2,
                                   C2.data_ptr(), N2, s, need2)

    say(f"[gpu] sgemm_ws_noalloc graph: eager {M}x{N}x{K}")
    assert call() == sg.OK
    torch.cuda.synchronize()
    want = C.clone()
    assert other() == sg.OK
    torch.cuda.synchronize()
    want2 = C2.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm up on the capture stream
        assert call() == sg.OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    say("[gpu] sgemm_ws_noalloc graph: capture")
    with torch.cuda.graph(graph):
        assert call() == sg.OK
    for rep in range(4):
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"[gpu] sgemm_ws_noalloc graph: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, want), rep
        # eager work between the replays: another split call through the scratch
        C2.fill_(float("nan"))
        assert other() == sg.OK
        torch.cuda.synchronize()
        assert torch.equal(C2, want2), rep
