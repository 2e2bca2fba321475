"""Compile the CPU oracle (test infrastructure) into ``oracle/liboracle.so``.

Flags keep the oracle a plain scalar program: no auto-vectorisation and no
fused multiply-add contraction, so every float operation rounds on its own.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zero_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-fno-tree-vectorize", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
