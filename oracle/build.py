"""Compile the CPU oracle (plain C, gcc, OpenMP) into oracle/libmoe_oracle.so.

Test infrastructure: the library built here is loaded only by the test suite,
the smoke check and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

# -ffp-contract=off: no fused multiply-adds, so every fp64 operation rounds once
# as written. No -ffast-math.
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall",
          "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
