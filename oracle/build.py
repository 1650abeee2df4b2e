"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Flags keep the arithmetic to plain IEEE-754 binary32/binary64 operations:
no contraction into fused multiply-add, no fast-math reassociation, SSE2
scalar floating point (no x87 excess precision).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dit_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FLAGS = [
    "-std=c11", "-O2", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-mfpmath=sse", "-msse2", "-Wall", "-Wextra",
]


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    cmd = ["gcc", *FLAGS, "-I", HERE, src, "-o", lib + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
