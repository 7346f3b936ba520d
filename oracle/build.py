"""Build the CPU oracle (liboracle.so) with gcc.

Test infrastructure only: the oracle is built beside the HIP library so the
checker exists, never linked into it.  Flags keep every fp32 step IEEE
round-to-nearest-even with no contraction and no fast-math, so the oracle's
quantization decisions are the ones its source states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
        "-fopenmp", "-Wall", "-Wextra", "-Wno-unused-parameter",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
