"""GPU parity: the HIP kernels, called through the C ABI, against the CPU
oracle on the same seeded inputs, |C - Cref| <= 1e-5 * (|A|·|B|) elementwise
(bit-exact where every partial sum is an integer)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import seedgen

from gpu_util import DevMat, assert_close, run, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ALGOS = ["auto", "mfma_direct", "mfma", "fma", "simple"]

# The five workloads: (name, M, N, K, lda, ldb, ldc, distribution, seed).
WORKLOAD_SHAPES = {
    "256cube": (256, 256, 256, 256, 256, 256, "uniform", 1),
    "4096cube": (4096, 4096, 4096, 4096, 4096, 4096, "uniform", 2),
    "ragged": (1000, 1500, 777, 777, 1500, 1500, "uniform", 3),
    "skinny": (65536, 128, 256, 256, 128, 128, "normal", 4),
    "8192cube": (8192, 8192, 8192, 8192, 8192, 8192, "normal", 5),
}

_inputs: dict = {}


def config_inputs(name):
    if name not in _inputs:
        M, N, K, lda, ldb, ldc, dist, seed = WORKLOAD_SHAPES[name]
        say(f"[inputs] {name}: M={M} N={N} K={K} {dist} seed={seed}")
        A, B = seedgen.gemm_inputs(M, N, K, dist, seed, lda=lda, ldb=ldb)
        _inputs[name] = (A, B, DevMat(A), DevMat(B))
    return _inputs[name]


@pytest.fixture(scope="module", autouse=True)
def _cleanup():
    yield
    _inputs.clear()


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("name", ["256cube", "ragged", "skinny"])
def test_config_full(name, algo):
    M, N, K, lda, ldb, ldc, dist, seed = WORKLOAD_SHAPES[name]
    A, B, dA, dB = config_inputs(name)
    dC = DevMat(np.full((M, ldc), np.nan, np.float32))
    say(f"[gpu] {name} algo={algo}")
    if not run(M, N, K, dA, dB, dC, algo):
        return
    Cref, T = oracle.gemm(A[:, :K], B[:, :N], M=M, N=N, K=K)
    err = assert_close(dC.host()[:, :N], Cref, T, f"{name}/{algo}")
    say(f"  max normalised error {err:.3e}")


def sample_indices(n: int, count: int, tile: int, seed: int) -> np.ndarray:
    """First, last, tile-boundary and seeded random indices in [0, n)."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, n - 1, n - 2] + [t for b in range(tile, n, tile * 7)
                                     for t in (b - 1, b)]
    rand = rng.choice(n, size=count, replace=False)
    return np.unique(np.clip(np.array(fixed + list(rand)), 0, n - 1))


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("name", ["4096cube", "8192cube"])
def test_config_sampled(name, algo):
    """Full-size shapes: the GPU computes all of C; the oracle computes every
    element of sampled rows and of sampled columns."""
    M, N, K, lda, ldb, ldc, dist, seed = WORKLOAD_SHAPES[name]
    A, B, dA, dB = config_inputs(name)
    dC = DevMat(np.full((M, ldc), np.nan, np.float32))
    say(f"[gpu] {name} algo={algo}")
    assert run(M, N, K, dA, dB, dC, algo)
    C = dC.host()
    assert np.all(np.isfinite(C[:, :N])), "unwritten or non-finite outputs"
    nsamp = 48 if M <= 4096 else 24
    rows = sample_indices(M, nsamp, 128, seed)
    cols = sample_indices(N, nsamp, 128, seed + 100)
    Cr, Tr = oracle.gemm(np.ascontiguousarray(A[rows, :K]), B[:, :N],
                         M=len(rows), N=N, K=K)
    assert_close(C[rows, :N], Cr, Tr, f"{name}/{algo} rows")
    Cc, Tc = oracle.gemm(A[:, :K], np.ascontiguousarray(B[:K, cols]),
                         M=M, N=len(cols), K=K)
    err = assert_close(C[:, cols], Cc, Tc, f"{name}/{algo} cols")
    say(f"  max normalised error (sampled) {err:.3e}")


SWEEP = [1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128,
         129, 255, 256, 257]


def int_case(M, N, K, seed, lda=None, ldb=None):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    A = np.full((M, lda), np.nan, np.float32)
    B = np.full((K, ldb), np.nan, np.float32)
    A[:, :K] = seedgen.integer_matrix(M, K, -8, 8, seed)
    B[:, :N] = seedgen.integer_matrix(K, N, -8, 8, seed, start=M * K)
    return A, B


@pytest.mark.parametrize("algo", ALGOS)
def test_integer_shapes_bitexact(algo):
    """Integer data: every partial sum is an integer below 2**24, so any
    summation order gives the same float32 bits as the rounded oracle."""
    rng = np.random.default_rng(7)
    shapes = [(m, n, k) for m in SWEEP for n in SWEEP for k in SWEEP]
    picks = [shapes[i] for i in rng.choice(len(shapes), 60, replace=False)]
    picks += [(1, 1, 1), (257, 257, 257), (1, 257, 3), (129, 1, 64),
              (1000, 1500, 777), (300, 500, 0)]
    for idx, (M, N, K) in enumerate(picks):
        A, B = int_case(M, N, K, 500 + idx)
        dA, dB = DevMat(A), DevMat(B)
        dC = DevMat(np.full((M, N), np.nan, np.float32))
        say(f"[gpu] int {algo} M={M} N={N} K={K}")
        if not run(M, N, K, dA, dB, dC, algo):
            continue
        Cref, _ = oracle.gemm(A[:, :K], B[:, :N], M=M, N=N, K=K, with_t=False)
        got = dC.host()
        assert np.array_equal(got, Cref.astype(np.float32)), (algo, M, N, K)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("offs", [(0, 0, 0), (1, 2, 3), (3, 1, 2), (2, 3, 1)])
def test_leading_dims_offsets_and_sentinels(algo, offs):
    """Leading dimensions wider than the rows (odd and multiple-of-4 ones),
    base addresses that are only 4-byte aligned, NaN in every A and B gap and
    sentinels in C's gaps, which must survive untouched."""
    for (M, N, K, lda, ldb, ldc) in [(130, 150, 77, 80, 151, 157),
                                     (200, 136, 96, 100, 140, 144),
                                     (65, 257, 33, 36, 260, 259)]:
        A, B = seedgen.gemm_inputs(M, N, K, "uniform", 900 + M, lda=lda,
                                   ldb=ldb, fill=np.nan)
        dA = DevMat(A, off=offs[0], pad=np.nan)
        dB = DevMat(B, off=offs[1], pad=np.nan)
        C0 = np.full((M, ldc), -123.5, np.float32)
        dC = DevMat(C0, off=offs[2], pad=-77.0)
        say(f"[gpu] ld {algo} offs={offs} M={M} N={N} K={K} ld={lda},{ldb},{ldc}")
        if not run(M, N, K, dA, dB, dC, algo):
            assert np.all(dC.host() == -123.5), "a refused call wrote C"
            continue
        got = dC.host()
        Cref, T = oracle.gemm(A[:, :K], B[:, :N], M=M, N=N, K=K)
        assert_close(got[:, :N], Cref, T, f"ld {algo} {offs}")
        assert np.all(got[:, N:] == -123.5), "C padding columns were written"
        w = dC.whole()
        assert np.all(w[:offs[2]] == -77.0)
        assert np.all(w[offs[2] + M * ldc:] == -77.0), "wrote past C"


@pytest.mark.parametrize("algo", ALGOS)
def test_deterministic_and_stream_independent(algo):
    M, N, K = 777, 556, 332
    A, B = seedgen.gemm_inputs(M, N, K, "normal", 77)
    dA, dB = DevMat(A), DevMat(B)
    outs = []
    s = torch.cuda.Stream()
    for stream in (None, None, s):
        dC = DevMat(np.zeros((M, N), np.float32))
        say(f"[gpu] determinism {algo} stream={'side' if stream else 'current'}")
        if stream is not None:
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                assert run(M, N, K, dA, dB, dC, algo, stream=stream)
        else:
            assert run(M, N, K, dA, dB, dC, algo)
        outs.append(dC.host().copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("algo", ALGOS)
def test_power_of_two_scaling_is_exact(algo):
    M, N, K = 300, 260, 192
    A, B = seedgen.gemm_inputs(M, N, K, "uniform", 88)
    dB = DevMat(B)
    res = []
    for scale in (1.0, 2.0, 0.25):
        dA = DevMat((A * np.float32(scale)).astype(np.float32))
        dC = DevMat(np.zeros((M, N), np.float32))
        say(f"[gpu] scaling {algo} x{scale}")
        assert run(M, N, K, dA, dB, dC, algo)
        res.append(dC.host().copy())
    assert np.array_equal(res[1], 2.0 * res[0])
    assert np.array_equal(res[2], 0.25 * res[0])


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("M,N,K", [(1000, 1500, 777), (333, 517, 129)])
def test_transposed_operands(algo, M, N, K):
    """(A·B)^T = B^T·A^T: the product of the transposed operands (made on the
    host) is the transpose of the product, within tolerance on random data
    and bit for bit on integer data, where every order of the sum is exact.
    The integer product is also transposed on the GPU by sgemm_transpose."""
    import tiled_fp32_gemm_amd as sg
    A, B = seedgen.gemm_inputs(M, N, K, "uniform", 97)
    dAt = DevMat(np.ascontiguousarray(A.T))
    dBt = DevMat(np.ascontiguousarray(B.T))
    dCt = DevMat(np.full((N, M), np.nan, np.float32))
    say(f"[gpu] transposed operands {algo} {M}x{N}x{K}")
    assert run(N, M, K, dBt, dAt, dCt, algo)
    Cref, T = oracle.gemm(A, B)
    assert_close(np.ascontiguousarray(dCt.host().T), Cref, T, f"(A.B)^T {algo}")

    Ai = seedgen.integer_matrix(M, K, -8, 8, 98)
    Bi = seedgen.integer_matrix(K, N, -8, 8, 98, start=M * K)
    dA, dB = DevMat(Ai), DevMat(Bi)
    dC = DevMat(np.full((M, N), np.nan, np.float32))
    assert run(M, N, K, dA, dB, dC, algo)
    dAt, dBt = DevMat(np.ascontiguousarray(Ai.T)), DevMat(np.ascontiguousarray(Bi.T))
    assert run(N, M, K, dBt, dAt, dCt, algo)
    dT = DevMat(np.full((N, M), np.nan, np.float32))
    assert sg.sgemm_transpose(M, N, dC.ptr, N, dT.ptr, M,
                              torch.cuda.current_stream().cuda_stream) == sg.OK
    torch.cuda.synchronize()
    assert np.array_equal(dT.host(), dCt.host())
    assert np.array_equal(dC.host(), oracle.gemm(Ai, Bi, with_t=False)[0].astype(np.float32))


@pytest.mark.parametrize("algo", ALGOS)
def test_k_zero_writes_zeros_and_empty_is_noop(algo):
    import tiled_fp32_gemm_amd as sg
    M, N = 70, 90
    dC = DevMat(np.full((M, N), 5.0, np.float32))
    say(f"[gpu] K=0 {algo}")
    st = sg.sgemm_ex(M, N, 0, 0, 1, 0, N, dC.ptr, N,
                     torch.cuda.current_stream().cuda_stream, sg.ALGOS[algo])
    assert st == sg.OK
    torch.cuda.synchronize()
    assert np.all(dC.host() == 0.0)
    dC2 = DevMat(np.full((4, 4), 5.0, np.float32))
    assert sg.sgemm_ex(0, 4, 4, 0, 4, 0, 4, dC2.ptr, 4, 0, sg.ALGOS[algo]) == sg.OK
    torch.cuda.synchronize()
    assert np.all(dC2.host() == 5.0)


# One shape per LDS-direct variant the planner can pick (the test checks the
# pick), each with K not a multiple of 4 so that the straddling A groups are
# zero-filled, and with an odd lda so that A rows are only 4-byte aligned.
VARIANT_SHAPES = [
    ("mfma_lds_256x256x32", 2048, 8192, 450),
    ("mfma_lds_128x128x32", 4096, 4096, 22),
    ("mfma_lds_64x128x32", 3072, 2048, 45),
    ("mfma_lds_64x128x32_ks2", 640, 3072, 42),
    ("mfma_lds_64x64x32", 1536, 3072, 47),
    ("mfma_lds_64x64x32_ks2", 3072, 192, 53),
    ("mfma_lds_32x64x32_ks2", 384, 4096, 61),
    ("mfma_lds_32x64x64_ks4", 32, 64, 67),
]


# (kernel, M, N, K): K a multiple of 4 that ends inside a slab, so in the last
# slab whole 4-float groups of A lie past k = K; with lda = K + 12 they are
# A's NaN padding columns, which the kernels must not let reach C.
K_TAIL_SHAPES = [
    ("mfma_lds_256x256x32", 4096, 8192, 52),
    ("mfma_lds_128x128x32", 1536, 8192, 148),
    ("mfma_lds_64x128x32", 1024, 4096, 452),
    ("mfma_lds_64x128x32_ks2", 640, 3072, 116),
    ("mfma_lds_64x64x32", 384, 8192, 452),
    ("mfma_lds_64x64x32_ks2", 192, 3072, 340),
    ("mfma_lds_32x64x32_ks2", 192, 8192, 452),
    ("mfma_lds_32x64x64_ks4", 32, 64, 452),
]


@pytest.mark.parametrize("kernel,M,N,K", K_TAIL_SHAPES, ids=[v[0] for v in K_TAIL_SHAPES])
def test_every_direct_variant_whole_groups_past_k(kernel, M, N, K):
    import tiled_fp32_gemm_amd as sg
    lda = K + 12
    A, B = seedgen.gemm_inputs(M, N, K, "uniform", 1800 + K, lda=lda, fill=np.nan)
    dA, dB = DevMat(A), DevMat(B)
    dC = DevMat(np.full((M, N), np.nan, np.float32))
    st, plan = sg.sgemm_plan_query(M, N, K, dA.ptr, lda, dB.ptr, N, dC.ptr, N, 0)
    assert st == sg.OK and plan.kernel.decode().rsplit("_", 1)[0] == kernel
    say(f"[gpu] K tail {kernel} M={M} N={N} K={K} lda={lda}")
    assert run(M, N, K, dA, dB, dC, "auto")
    Cref, T = oracle.gemm(A[:, :K], B, M=M, N=N, K=K)
    assert_close(dC.host(), Cref, T, f"K tail {kernel}")


# (kernel, M, N, K): one, two and three slabs, the last one partial, so that
# each variant runs its single-slab path, the peeled step with no loads, and
# one step with loads before it (integer data: every order gives the same
# bits).
SHORT_K_SHAPES = [
    ("mfma_lds_128x128x32", 637, 4101, 9),
    ("mfma_lds_128x128x32", 381, 8197, 51),
    ("mfma_lds_128x128x32", 381, 8197, 83),
    ("mfma_lds_64x128x32", 637, 8197, 9),
    ("mfma_lds_64x128x32", 637, 8197, 51),
    ("mfma_lds_64x128x32", 637, 8197, 83),
    ("mfma_lds_64x128x32_ks2", 1533, 645, 9),
    ("mfma_lds_64x128x32_ks2", 189, 8197, 51),
    ("mfma_lds_64x128x32_ks2", 189, 8197, 83),
    ("mfma_lds_64x64x32", 4093, 389, 9),
    ("mfma_lds_64x64x32", 4093, 389, 51),
    ("mfma_lds_64x64x32", 4093, 389, 83),
    ("mfma_lds_64x64x32_ks2", 32, 37, 9),
    ("mfma_lds_64x64x32_ks2", 3069, 133, 51),
    ("mfma_lds_64x64x32_ks2", 3069, 133, 83),
    ("mfma_lds_32x64x32_ks2", 32, 1029, 9),
    ("mfma_lds_32x64x32_ks2", 6141, 133, 51),
    ("mfma_lds_32x64x32_ks2", 93, 8197, 83),
    ("mfma_lds_32x64x64_ks4", 32, 37, 99),
    ("mfma_lds_32x64x64_ks4", 32, 37, 163),
]


@pytest.mark.parametrize("kernel,M,N,K", SHORT_K_SHAPES,
                         ids=[f"{v[0]}-K{v[3]}" for v in SHORT_K_SHAPES])
def test_every_direct_variant_one_to_three_slabs(kernel, M, N, K):
    import tiled_fp32_gemm_amd as sg
    lda, ldc = K + 1, N + 2
    A = np.full((M, lda), np.nan, np.float32)
    A[:, :K] = seedgen.integer_matrix(M, K, -8, 8, 2100 + K)
    B = seedgen.integer_matrix(K, N, -8, 8, 2100 + K, start=M * K)
    dA, dB = DevMat(A), DevMat(B)
    dC = DevMat(np.full((M, ldc), np.nan, np.float32))
    st, plan = sg.sgemm_plan_query(M, N, K, dA.ptr, lda, dB.ptr, N, dC.ptr, ldc, 0)
    assert st == sg.OK and plan.kernel.decode().rsplit("_", 1)[0] == kernel
    say(f"[gpu] short K {kernel} M={M} N={N} K={K}")
    st = sg.sgemm(M, N, K, dA.ptr, lda, dB.ptr, N, dC.ptr, ldc,
                  torch.cuda.current_stream().cuda_stream)
    assert st == sg.OK
    torch.cuda.synchronize()
    C = dC.host()
    Cref, _ = oracle.gemm(A[:, :K], B, M=M, N=N, K=K, with_t=False)
    assert np.array_equal(C[:, :N], Cref.astype(np.float32))
    assert np.all(np.isnan(C[:, N:])), "C padding written"


# (kernel, M, N, K): tiles with two 32-column blocks per wave store C as
# column pairs, and a tile on C's right edge takes its own path that stores
# each word under its own mask.  N leaves an odd number of columns in the
# last tile column (5 or 37), so a lane there holds one valid column of its
# pair, and whole waves of the tile lie past N.  Integer data: every order
# gives the same bits; C's padding columns must stay untouched.
PAIR_EDGE_SHAPES = [
    ("mfma_lds_256x256x32", 4096, 3845, 1200),
    ("mfma_lds_256x256x32", 3840, 4133, 1000),
    ("mfma_lds_128x128x32", 4096, 4101, 64),
    ("mfma_lds_64x128x32", 4096, 4101, 256),
]


@pytest.mark.parametrize("kernel,M,N,K", PAIR_EDGE_SHAPES,
                         ids=[f"{v[0]}-{v[1]}x{v[2]}x{v[3]}" for v in PAIR_EDGE_SHAPES])
def test_paired_columns_at_the_right_edge(kernel, M, N, K):
    import tiled_fp32_gemm_amd as sg
    lda, ldc = K + 1, N + 2
    A = np.full((M, lda), np.nan, np.float32)
    A[:, :K] = seedgen.integer_matrix(M, K, -8, 8, 2300 + K)
    B = seedgen.integer_matrix(K, N, -8, 8, 2300 + K, start=M * K)
    dA, dB = DevMat(A), DevMat(B)
    dC = DevMat(np.full((M, ldc), np.nan, np.float32))
    st, plan = sg.sgemm_plan_query(M, N, K, dA.ptr, lda, dB.ptr, N, dC.ptr, ldc, 0)
    assert st == sg.OK and plan.kernel.decode().rsplit("_", 1)[0] == kernel
    say(f"[gpu] paired-column edge {kernel} M={M} N={N} K={K}")
    st = sg.sgemm(M, N, K, dA.ptr, lda, dB.ptr, N, dC.ptr, ldc,
                  torch.cuda.current_stream().cuda_stream)
    assert st == sg.OK
    torch.cuda.synchronize()
    C = dC.host()
    Cref, _ = oracle.gemm(A[:, :K], B, M=M, N=N, K=K, with_t=False)
    assert np.array_equal(C[:, :N], Cref.astype(np.float32))
    assert np.all(np.isnan(C[:, N:])), "C padding written"


@pytest.mark.parametrize("kernel,M,N,K", VARIANT_SHAPES, ids=[v[0] for v in VARIANT_SHAPES])
@pytest.mark.parametrize("odd_lda", [False, True])
def test_every_direct_variant(kernel, M, N, K, odd_lda):
    import tiled_fp32_gemm_amd as sg
    lda = K + (3 if odd_lda else 1)
    A, B = seedgen.gemm_inputs(M, N, K, "uniform", 1700 + K, lda=lda, fill=np.nan)
    dA, dB = DevMat(A), DevMat(B)
    dC = DevMat(np.full((M, N), np.nan, np.float32))
    st, plan = sg.sgemm_plan_query(M, N, K, dA.ptr, lda, dB.ptr, N, dC.ptr, N, 0)
    assert st == sg.OK and plan.kernel.decode().rsplit("_", 1)[0] == kernel
    say(f"[gpu] variant {kernel} M={M} N={N} K={K} lda={lda}")
    assert run(M, N, K, dA, dB, dC, "auto")
    Cref, T = oracle.gemm(A[:, :K], B, M=M, N=N, K=K)
    assert_close(dC.host(), Cref, T, kernel)


def test_matmul_wrapper_on_views():
    """The tensor convenience: row-stride views and the current stream."""
    import tiled_fp32_gemm_amd as sg
    M, N, K = 123, 77, 45
    A, B = seedgen.gemm_inputs(M, N, K, "uniform", 99)
    big = torch.full((M, K + 11), float("nan"), device="cuda:0")
    big[:, :K] = torch.from_numpy(A)
    tA = big[:, :K]
    tB = torch.from_numpy(B).to("cuda:0")
    say("[gpu] matmul wrapper")
    out = sg.matmul(tA, tB)
    torch.cuda.synchronize()
    Cref, T = oracle.gemm(A, B)
    assert_close(out.cpu().numpy(), Cref, T, "matmul")
    with pytest.raises(ValueError):
        sg.matmul(tA.double(), tB)
    with pytest.raises(ValueError):
        sg.matmul(tA.t(), tB)
