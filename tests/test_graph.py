"""The library's launches under HIP graph capture: sgemm, sgemm_ws (K split
across workgroups, two kernels through a workspace) and sgemm_transpose
enqueue only kernel launches (no memsets, no allocation, no synchronisation),
so a captured sequence replays to the same bits as the eager calls.  The
graph is replayed several times with eager work and synchronisation between
the replays, and every replay is checked."""
from __future__ import annotations

import numpy as np
import pytest

import seedgen

from gpu_util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SHAPES = [(4096, 4096, 512), (1000, 1500, 777), (65536, 128, 256), (256, 256, 256)]


def test_captured_products_replay_bit_exact():
    import tiled_fp32_gemm_amd as sg
    dev = torch.device("cuda:0")
    ops = []
    for idx, (M, N, K) in enumerate(SHAPES):
        A, B = seedgen.gemm_inputs(M, N, K, "normal", 1300 + idx)
        ops.append((M, N, K, torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                    torch.empty((M, N), device=dev)))
    # split products: (M, N, K, A, B, C), one workspace shared in stream order
    splits = []
    for idx, (M, N, K) in enumerate([(256, 256, 8192), (200, 300, 10001)]):
        A, B = seedgen.gemm_inputs(M, N, K, "normal", 1350 + idx)
        assert sg.sgemm_workspace_bytes(M, N, K) > 0
        splits.append((M, N, K, torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                       torch.empty((M, N), device=dev)))
    ws_bytes = max(sg.sgemm_workspace_bytes(M, N, K) for M, N, K, *_ in splits)
    ws = torch.empty(ws_bytes // 4, device=dev)
    tin = torch.rand((1000, 1500), device=dev)
    tout = torch.empty((1500, 1000), device=dev)

    def enqueue():
        s = torch.cuda.current_stream().cuda_stream
        for M, N, K, tA, tB, tC in ops:
            assert sg.sgemm(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N,
                            tC.data_ptr(), N, s) == sg.OK
        for M, N, K, tA, tB, tC in splits:
            assert sg.sgemm_ws(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N,
                               tC.data_ptr(), N, s, ws.data_ptr(), ws_bytes) == sg.OK
        assert sg.sgemm_transpose(1000, 1500, tin.data_ptr(), 1500,
                                  tout.data_ptr(), 1000, s) == sg.OK

    say("[gpu] graph: eager reference")
    enqueue()
    torch.cuda.synchronize()
    outs = ops + splits
    want = [op[5].clone() for op in outs] + [tout.clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm up on the capture stream
        enqueue()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    say("[gpu] graph: capture")
    with torch.cuda.graph(graph):
        enqueue()
    for rep in range(4):
        for op in outs:
            op[5].fill_(float("nan"))
        ws.fill_(float("nan"))
        tout.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"[gpu] graph: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        got = [op[5] for op in outs] + [tout]
        for w, g in zip(want, got):
            assert torch.equal(w, g), rep
        # eager work of the program between the replays
        junk = torch.randn((512, 512), device=dev) @ torch.randn((512, 512), device=dev)
        torch.cuda.synchronize()
        assert torch.isfinite(junk).all()
