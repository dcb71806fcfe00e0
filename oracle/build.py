"""Build the CPU oracle library (test infrastructure only).

    python oracle/build.py

Compiles hardkv_oracle.c with gcc at -O2, with floating-point contraction
disabled and no fast-math, so that every float operation rounds once.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hardkv_oracle.c")
LIB = os.path.join(HERE, "liboracle_hardkv.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
