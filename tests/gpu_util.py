"""Helpers for the GPU tests: device buffers with chosen leading dimensions
and base offsets, calls through the C ABI, and the acceptance check."""
from __future__ import annotations

import sys

import numpy as np

import tiled_fp32_gemm_amd as sg

TOL = 1e-5   # |C - Cref| <= TOL * (|A|·|B|), elementwise


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class DevMat:
    """A rows x ld float32 device buffer whose first element sits ``off``
    floats into a fresh allocation (so its address can be 4-byte aligned
    only).  The padding floats before and after are filled with ``pad``."""

    def __init__(self, host: np.ndarray, off: int = 0, pad: float = np.nan,
                 device: str = "cuda:0"):
        import torch
        assert host.dtype == np.float32 and host.ndim == 2
        self.rows, self.ld = host.shape
        n = self.rows * self.ld
        flat = np.full(off + n + 4, pad, dtype=np.float32)
        flat[off:off + n] = host.ravel()
        self.buf = torch.from_numpy(flat).to(device)
        self.off = off

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + 4 * self.off

    def host(self) -> np.ndarray:
        flat = self.buf.cpu().numpy()
        return flat[self.off:self.off + self.rows * self.ld].reshape(
            self.rows, self.ld)

    def whole(self) -> np.ndarray:
        return self.buf.cpu().numpy()


def vec_rows(ptr: int, ld: int, width: int) -> bool:
    """Rows that allow 128-bit loads: 16-byte base, ld and width % 4 == 0."""
    return ptr % 16 == 0 and ld % 4 == 0 and width % 4 == 0


def run(M, N, K, dA: DevMat, dB: DevMat, dC: DevMat, algo="auto",
        stream=None, sync=True) -> bool:
    """One call through the C ABI; True once the product has run."""
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    st = sg.sgemm_ex(M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr, dC.ld,
                     s.cuda_stream, sg.ALGOS[algo])
    assert st == sg.OK, sg.sgemm_status_string(st)
    if sync:
        torch.cuda.synchronize()
    return True


def max_norm_err(C: np.ndarray, Cref: np.ndarray, T: np.ndarray) -> float:
    d = np.abs(C.astype(np.float64) - Cref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(T > 0, d / T, np.where(d > 0, np.inf, 0.0))
    return float(r.max()) if r.size else 0.0


def assert_close(C: np.ndarray, Cref: np.ndarray, T: np.ndarray,
                 what: str = "") -> float:
    """Every element within TOL * T of the oracle (exact where T == 0)."""
    assert C.shape == Cref.shape == T.shape
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"
    err = np.abs(C.astype(np.float64) - Cref)
    bad = err > TOL * T
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} elements out of tolerance; first at "
            f"({i},{j}): got {C[i, j]!r}, oracle {Cref[i, j]!r}, T {T[i, j]!r}")
    return max_norm_err(C, Cref, T)
