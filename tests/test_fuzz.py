"""Seeded random ragged shapes through every family and the split path.

Shapes are drawn log-uniformly (M, N up to 3000 for the planner's paths and
1500 for the fixed families, K up to 1200; half of them at least 200 a side;
a third with K near a slab boundary), with leading dimensions up to 4 floats
past the row, base addresses 0-3 floats into their allocation, and NaN in
every padding float of A and B.  Integer data in [-8, 8], so every
summation order gives the same bits: C must equal the oracle's rounded
product bit for bit, and C's padding columns must stay untouched ("CUDA in
depth (5): vectorized load and shared-memory layout", sections on edges and
on leading dimensions).  Every call goes through the C ABI; the planner's
picks are printed, so the run shows which kernels it covered.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import seedgen
from gpu_util import DevMat, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SLAB_EDGES = [1, 2, 3, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129]


def shapes(seed: int, n: int, top: int = 1500):
    rs = np.random.RandomState(seed)
    out = []
    for _ in range(n):
        # half the shapes from 1 up, half from 200 up (several tiles a side)
        lo = 0.0 if rs.rand() < 0.5 else np.log(200)
        M, N = (int(np.exp(rs.uniform(lo, np.log(top)))) for _ in range(2))
        K = int(np.exp(rs.uniform(lo, np.log(1200))))
        if rs.rand() < 0.3:
            K = int(rs.choice(SLAB_EDGES))
        pads = [int(x) for x in rs.randint(0, 5, 3)]
        offs = [int(x) for x in rs.randint(0, 4, 3)]
        out.append((M, N, K, pads, offs))
    return out


@pytest.mark.parametrize("algo", ["auto", "mfma", "fma", "simple", "ws"])
def test_random_ragged_shapes_bitexact(algo):
    import tiled_fp32_gemm_amd as sg
    stream = torch.cuda.current_stream().cuda_stream
    ws = torch.empty(16 << 20, device="cuda:0")     # 64 MiB
    picks = {}
    # the planner's families see larger shapes (more of its tile choices)
    cases = (shapes(4242, 100, 3000) if algo in ("auto", "ws") else
             shapes(4242, 40 if algo != "simple" else 15))
    for it, (M, N, K, (pa, pb, pc), (oa, ob, oc)) in enumerate(cases):
        lda, ldb, ldc = K + pa, N + pb, N + pc
        A = np.full((M, lda), np.nan, np.float32)
        B = np.full((K, ldb), np.nan, np.float32)
        A[:, :K] = seedgen.integer_matrix(M, K, -8, 8, 3000 + it)
        B[:, :N] = seedgen.integer_matrix(K, N, -8, 8, 3000 + it, start=M * K)
        dA, dB = DevMat(A, off=oa), DevMat(B, off=ob)
        dC = DevMat(np.full((M, ldc), np.nan, np.float32), off=oc)
        if algo == "ws":
            nb = ws.numel() * 4
            st, plan = sg.sgemm_plan_query_ws(M, N, K, dA.ptr, lda, dB.ptr, ldb, dC.ptr,
                                              ldc, nb)
            assert st == sg.OK
            say(f"[gpu] fuzz {algo} #{it} {M}x{N}x{K} ld={lda},{ldb},{ldc} "
                f"off={oa},{ob},{oc} {plan.kernel.decode()}")
            st = sg.sgemm_ws(M, N, K, dA.ptr, lda, dB.ptr, ldb, dC.ptr, ldc, stream,
                             ws.data_ptr(), nb)
        else:
            st, plan = sg.sgemm_plan_query(M, N, K, dA.ptr, lda, dB.ptr, ldb, dC.ptr, ldc,
                                           sg.ALGOS[algo])
            assert st == sg.OK
            say(f"[gpu] fuzz {algo} #{it} {M}x{N}x{K} ld={lda},{ldb},{ldc} "
                f"off={oa},{ob},{oc} {plan.kernel.decode()}")
            st = sg.sgemm_ex(M, N, K, dA.ptr, lda, dB.ptr, ldb, dC.ptr, ldc, stream,
                             sg.ALGOS[algo])
        assert st == sg.OK, sg.sgemm_status_string(st)
        torch.cuda.synchronize()
        C = dC.host()
        Cref, _ = oracle.gemm(A[:, :K], B[:, :N], M=M, N=N, K=K, with_t=False)
        assert np.array_equal(C[:, :N], Cref.astype(np.float32)), (algo, it, M, N, K)
        assert np.all(np.isnan(C[:, N:])), ("C padding written", algo, it)
        name = plan.kernel.decode()
        picks[name] = picks.get(name, 0) + 1
    say(f"  {algo}: {len(cases)} shapes, kernels: {dict(sorted(picks.items()))}")
