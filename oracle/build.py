"""Builds the CPU oracle (test infrastructure) as oracle/libmoe_ref.so with gcc.

Plain C, -O2 -fopenmp, no FMA contraction and no fast-math so each written
fp32 operation is one IEEE operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe_ref.so")


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """sanitize: AddressSanitizer + UndefinedBehaviorSanitizer instrumentation
    (-O1 -g; the process that loads it needs the sanitizer runtimes
    preloaded), for the sanitizer test; out names that build's file."""
    src = os.path.join(HERE, "moe_ref.c")
    opt = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
    cmd = ["gcc", "-std=c11", *opt, "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter",
           src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
