"""GPU parity of the tiled transpose (sgemm_transpose*), bit for bit against
the CPU oracle, through the C ABI, for every LDS layout."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import seedgen

from gpu_util import DevMat, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LAYOUTS = ["auto", "naive", "padded", "swizzled"]


def run_t(rows, cols, dIn: DevMat, dOut: DevMat, layout: str) -> None:
    import tiled_fp32_gemm_amd as sg
    st = sg.sgemm_transpose_ex(rows, cols, dIn.ptr, dIn.ld, dOut.ptr, dOut.ld,
                               torch.cuda.current_stream().cuda_stream,
                               sg.TRANSPOSE_LAYOUTS[layout])
    assert st == sg.OK, sg.sgemm_status_string(st)
    torch.cuda.synchronize()


SHAPES = [(1, 1), (1, 257), (257, 1), (63, 65), (64, 64), (65, 63), (100, 200),
          (128, 4), (4, 128), (64, 128), (65, 129), (63, 127), (127, 255),
          (1000, 1500), (777, 4099), (2048, 64)]


@pytest.mark.parametrize("layout", LAYOUTS)
def test_shapes_bitexact(layout):
    for idx, (r, c) in enumerate(SHAPES):
        A = seedgen.matrix(r, c, "normal", 300 + idx)
        dIn = DevMat(A)
        dOut = DevMat(np.full((c, r), np.nan, np.float32))
        say(f"[gpu] transpose {layout} {r}x{c}")
        run_t(r, c, dIn, dOut, layout)
        assert np.array_equal(dOut.host(), oracle.transpose(A)), (layout, r, c)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("offs", [(0, 0), (1, 3), (2, 1), (3, 2)])
def test_leading_dims_offsets_sentinels(layout, offs):
    r, c = 131, 97
    A = seedgen.matrix(r, c, "uniform", 77, ld=c + 5, fill=np.nan)
    dIn = DevMat(A, off=offs[0], pad=np.nan)
    dOut = DevMat(np.full((c, r + 3), -9.0, np.float32), off=offs[1], pad=-4.0)
    say(f"[gpu] transpose ld {layout} offs={offs}")
    run_t(r, c, dIn, dOut, layout)
    got = dOut.host()
    want = oracle.transpose(A[:, :c], rows=r, cols=c, ldo=r + 3, fill=-9.0)
    assert np.array_equal(got, want)
    w = dOut.whole()
    assert np.all(w[:offs[1]] == -4.0) and np.all(w[offs[1] + c * (r + 3):] == -4.0)


def test_empty_is_a_noop():
    import tiled_fp32_gemm_amd as sg
    dOut = DevMat(np.full((4, 4), 2.0, np.float32))
    assert sg.sgemm_transpose(0, 4, 0, 4, dOut.ptr, 4, 0) == sg.OK
    assert sg.sgemm_transpose(4, 0, 0, 1, dOut.ptr, 4, 0) == sg.OK
    torch.cuda.synchronize()
    assert np.all(dOut.host() == 2.0)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_large_sampled(layout):
    """8192 x 8192 (256 MiB each way): the oracle transposes sampled row
    blocks; every output element is checked finite."""
    import tiled_fp32_gemm_amd as sg
    r = c = 8192
    g = torch.Generator(device="cuda:0")
    g.manual_seed(5)
    tin = torch.rand((r, c), device="cuda:0", generator=g)
    tout = torch.full((c, r), float("nan"), device="cuda:0")
    say(f"[gpu] transpose large {layout}")
    st = sg.sgemm_transpose_ex(r, c, tin.data_ptr(), c, tout.data_ptr(), r,
                               torch.cuda.current_stream().cuda_stream,
                               sg.TRANSPOSE_LAYOUTS[layout])
    assert st == sg.OK
    torch.cuda.synchronize()
    assert bool(torch.isfinite(tout).all())
    for i0 in (0, 4032, 8128):
        blk = tin[i0:i0 + 64].cpu().numpy()
        assert np.array_equal(tout[:, i0:i0 + 64].cpu().numpy(), oracle.transpose(blk))


def test_tensor_wrapper():
    import tiled_fp32_gemm_amd as sg
    A = seedgen.matrix(50, 70, "normal", 9)
    t = torch.from_numpy(A).to("cuda:0")
    out = sg.transpose(t)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.transpose(A))
