"""Build the C++ oracle (test infrastructure) into oracle/c/liboracle_c.so with the host compiler.

    python -m oracle.c.build

Plain C++17, OpenMP over output rows, no floating-point contraction or fast-math, so every
rounding is the one written in the source."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gq8_oracle.cpp")
LIB = os.path.join(HERE, "liboracle_c.so")
CXX = shutil.which("g++") or "g++"
FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
         "-fvisibility=hidden"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [CXX, *FLAGS, SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
