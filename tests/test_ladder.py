"""GPU parity of every ablation ladder step (sgemm_ladder) against the CPU
oracle: bit-exact on integer data, within 1e-5 (|A|·|B|) on random data, on
shapes with ragged tiles, unaligned rows (the 128-bit steps fall back to
32-bit loads) and NaN-filled padding that must never be read."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import seedgen

from gpu_util import DevMat, assert_close, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_STEPS = 14


def ladder(step, M, N, K, dA, dB, dC):
    import tiled_fp32_gemm_amd as sg
    st = sg.sgemm_ladder(step, M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr,
                         dC.ld, torch.cuda.current_stream().cuda_stream)
    assert st == sg.OK, sg.sgemm_status_string(st)
    torch.cuda.synchronize()


def test_step_count_and_names():
    import tiled_fp32_gemm_amd as sg
    names = sg.ladder_steps()
    assert len(names) == N_STEPS and len(set(names)) == N_STEPS
    assert sg.sgemm_ladder_name(N_STEPS) is None and sg.sgemm_ladder_name(-1) is None


@pytest.mark.parametrize("step", range(N_STEPS))
def test_integer_data_bitexact(step):
    # (M, N, K, lda, ldb): ragged in every dimension; aligned rows, then
    # rows of A and B that are only 4-byte aligned
    for idx, (M, N, K, lda, ldb) in enumerate([(300, 260, 200, 200, 260),
                                               (129, 131, 97, 101, 133),
                                               (1, 70, 5, 5, 70),
                                               (64, 1, 33, 35, 1)]):
        A = np.full((M, lda), np.nan, np.float32)
        B = np.full((K, ldb), np.nan, np.float32)
        A[:, :K] = seedgen.integer_matrix(M, K, -8, 8, 900 + idx)
        B[:, :N] = seedgen.integer_matrix(K, N, -8, 8, 900 + idx, start=M * K)
        dA, dB = DevMat(A), DevMat(B)
        dC = DevMat(np.full((M, N), np.nan, np.float32))
        say(f"[gpu] ladder step {step} int M={M} N={N} K={K} lda={lda}")
        ladder(step, M, N, K, dA, dB, dC)
        Cref, _ = oracle.gemm(A[:, :K], B[:, :N], M=M, N=N, K=K, with_t=False)
        assert np.array_equal(dC.host(), Cref.astype(np.float32)), (step, M, N, K)


@pytest.mark.parametrize("step", range(N_STEPS))
def test_random_data_within_tolerance(step):
    M, N, K = 520, 392, 300
    A, B = seedgen.gemm_inputs(M, N, K, "normal", 950 + step)
    dA, dB = DevMat(A), DevMat(B)
    dC = DevMat(np.full((M, N), np.nan, np.float32))
    say(f"[gpu] ladder step {step} normal M={M} N={N} K={K}")
    ladder(step, M, N, K, dA, dB, dC)
    Cref, T = oracle.gemm(A, B)
    assert_close(dC.host(), Cref, T, f"ladder step {step}")


def test_zero_k_writes_zeros():
    for step in range(N_STEPS):
        M, N = 40, 70
        dA = DevMat(np.zeros((M, 1), np.float32))
        dB = DevMat(np.zeros((1, N), np.float32))
        dC = DevMat(np.full((M, N), np.nan, np.float32))
        say(f"[gpu] ladder step {step} K=0")
        ladder(step, M, N, 0, dA, dB, dC)
        assert np.all(dC.host() == 0.0), step
