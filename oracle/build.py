"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so.

gcc -O2 with floating-point contraction off and no fast-math, so that every
binary32 operation in the oracle rounds once and fmaf() is the only fused
operation; OpenMP parallelises over independent rows only.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
        "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
        "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
