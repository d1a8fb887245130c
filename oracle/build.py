"""Build the fp64 C oracle (test infrastructure) into oracle/libkda_oracle.so.

Plain gcc with OpenMP.  Nothing from the HIP library is compiled or linked in.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle; returns the path of the shared library."""
    tmp = LIB + ".tmp"
    # -ffp-contract=off keeps every multiply and add a separately rounded fp64
    # operation, so the oracle's arithmetic is exactly what its source says.
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Werror",
           "-std=c99", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
