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


CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile `src` (the oracle, or a copy of it) into the shared library `lib`."""
    cmd = ["gcc", *CFLAGS, "-o", lib + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
