"""Builds the CPU oracle (test infrastructure) as oracle/libmoe_ref.so with gcc.

Plain C, -O2 -fopenmp, no FMA contraction and no fast-math so each written
fp32 operation is one IEEE operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe_ref.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "moe_ref.c")
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter",
           src, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
