"""Compile the CPU oracle (test infrastructure) into oracle/libzpq_ref.so.

Plain gcc, single translation unit.  -ffp-contract=off keeps every float
expression as separately rounded IEEE binary32 operations (no fused
multiply-add), and no -ffast-math keeps IEEE division, signed zeros and
subnormals.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zpq_ref.c")
LIB = os.path.join(HERE, "libzpq_ref.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
