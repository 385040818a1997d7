"""Builds liboracle.so from oracle.c with gcc (-O2 -fopenmp, no fast-math).

Test infrastructure: the library it builds is loaded only by the tests, the
smoke check and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def compile_source(src: str, out: str, verbose: bool = False) -> str:
    """gcc ``src`` into the shared library ``out`` with the oracle's flags."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (always recompiles)."""
    return compile_source(SRC, LIB, verbose)


def ensure_built() -> str:
    """Build only when the library is missing or older than its source."""
    if (not os.path.exists(LIB)
            or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
        return build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
