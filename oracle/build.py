"""Build the CPU oracle shared library (test infrastructure only).

gcc, fp64, OpenMP. Targets x86-64-v3 (AVX2/FMA) so the library built in one
container also runs on another host of the same generation or newer.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    if (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
