"""Build the CPU oracle (test infrastructure) as a shared library with gcc.

Usage: python oracle/build.py   -> oracle/libprism_oracle.so
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "prism_oracle.c")
LIB = os.path.join(HERE, "libprism_oracle.so")

# Strict IEEE: no contraction of a*b+c into FMA, no fast-math, no vector intrinsics.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
