"""Python binding of the benchmark's measurement aids (``include/sgemm_probe.h``,
``libsgemm_probe.so``): argument marshalling only.

``mfma_clock(stream, iters, stamps)`` enqueues the fixed-work FP32
matrix-core kernel whose duration gives the clock the matrix pipes ran at;
``versions()`` returns the wall-clock rate and the HIP runtime and driver
versions.  Like the product binding, it raises if the library is missing.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsgemm_probe.so")
_lib = None

# From include/sgemm_probe.h.
WORKGROUPS = 256
WAVES = 16
MFMA_PER_ITER = 16
MFMA_CYCLES = 64
STAMP_WORDS = 5


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m tiled_fp32_gemm_amd.build`")
    import torch  # noqa: F401  (the HIP runtime torch ships is bound first)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.sgemm_probe_mfma_clock.argtypes = [ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_void_p]
    lib.sgemm_probe_mfma_clock.restype = ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int)
    lib.sgemm_probe_versions.argtypes = [ip, ip, ip]
    lib.sgemm_probe_versions.restype = ctypes.c_int
    _lib = lib
    return lib


def mfma_clock(stream: int, iters: int, stamps: int) -> int:
    """Enqueue the clock probe; ``stamps`` is a device address of
    ``STAMP_WORDS * WORKGROUPS`` uint64.  Returns the status code."""
    return load().sgemm_probe_mfma_clock(stream, iters, stamps)


def versions() -> dict:
    """``{"wall_clock_khz", "hip_runtime", "hip_driver"}`` of the current
    device (raises RuntimeError when HIP reports an error)."""
    w, r, d = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    st = load().sgemm_probe_versions(ctypes.byref(w), ctypes.byref(r),
                                     ctypes.byref(d))
    if st != 0:
        raise RuntimeError(f"sgemm_probe_versions failed (status {st})")
    return {"wall_clock_khz": w.value, "hip_runtime": r.value, "hip_driver": d.value}
