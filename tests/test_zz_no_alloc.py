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
