"""Compile the fp64 CPU oracle into oracle/liboracle.so with gcc.

Test infrastructure: the oracle checks the GPU library and is never part of it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "arp_oracle.c")
TARGET = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Always recompile; return the path of the shared library."""
    tmp = TARGET + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           SOURCE, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, TARGET)
    return TARGET


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
