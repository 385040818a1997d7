"""Builds libsgemm.so (the HIP kernels and the C ABI) and libsgemm_probe.so
(the benchmark's clock probe) for gfx950 with hipcc.

``python -m tiled_fp32_gemm_amd.build [--asm]`` compiles in-tree; ``--asm``
also writes the device assembly next to the sources' build folder
(``_build/``) for instruction counts.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsgemm.so")
PROBE_LIB = os.path.join(HERE, "libsgemm_probe.so")
ROOT = os.path.dirname(HERE)
ASM_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

# Packed FP32 instructions are kept out of the generated code (the vector
# kernels use single fused multiply-adds; the matrix kernels do not need them).
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-ffp-contract=fast", "-Wall"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) +
                  glob.glob(os.path.join(CSRC, "*.hpp")) +
                  glob.glob(os.path.join(ROOT, "include", "*.h")))


def _compile(src: str, out: str, verbose: bool) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["hipcc", *DEVICE_FLAGS, "-fPIC", "-shared",
           "-Wl,-rpath,/opt/rocm/lib", src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile ``csrc/sgemm.hip`` into ``libsgemm.so`` and ``csrc/probe.hip``
    into ``libsgemm_probe.so`` (always recompiles)."""
    _compile(os.path.join(CSRC, "probe.hip"), PROBE_LIB, verbose)
    return _compile(os.path.join(CSRC, "sgemm.hip"), LIB, verbose)


def build_asm() -> str:
    """Device assembly of the library, for reading our own instruction mix."""
    os.makedirs(ASM_DIR, exist_ok=True)
    out = os.path.join(ASM_DIR, f"sgemm-{ARCH}.s")
    cmd = ["hipcc", *DEVICE_FLAGS, "--offload-device-only", "-S",
           os.path.join(CSRC, "sgemm.hip"), "-o", out]
    subprocess.run(cmd, check=True)
    return out


def ensure_built() -> str:
    """Build only when a library is missing or older than a source."""
    newest = max(os.path.getmtime(s) for s in sources())
    if any(not os.path.exists(p) or os.path.getmtime(p) < newest
           for p in (LIB, PROBE_LIB)):
        return build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    if "--asm" in sys.argv:
        print(build_asm())
