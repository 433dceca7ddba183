"""Build the C part of the oracle (test infrastructure only).

`python -m oracle.build` or `oracle.build.build()` compiles gemm_ref.c with
gcc into oracle/_liborc.so.  The flags keep every rounding of the plain
definition: no fused multiply-add contraction and no fast-math.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_ref.c")
LIB = os.path.join(HERE, "_liborc.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
