"""Build the CPU oracle (test infrastructure) as oracle/liboracle.so with gcc.

Plain C11, -O2, OpenMP, IEEE semantics kept: no fast-math and no floating-
point contraction, so every fp32/fp64 operation rounds once, as written.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-frounding-math", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", OUT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
