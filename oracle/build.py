"""Compile the CPU oracle (oracle.c) into liboracle.so with gcc.

Test infrastructure: the oracle checks the HIP library and is never called by
it. Flags: -O2 without -ffast-math, -ffp-contract=off so that no fused
multiply-add changes the fixed summation order, OpenMP for the outer loops.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def compile_c(src: str, out: str, verbose: bool = False) -> str:
    """Compile one C file into a shared library at ``out`` (atomically)."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    return compile_c(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
