"""Build the CPU oracle (liboracle.so) with gcc.

TEST INFRASTRUCTURE ONLY: the oracle is what the HIP path is checked against.
Flags pin the arithmetic: -O2 without fast-math and with FMA contraction off,
so each fp32 operation in oracle.c is one IEEE-754 rounding.  -fopenmp turns
on the work-sharing pragmas over independent outputs (results do not depend
on the thread count).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "oracle.c")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
        "-fno-tree-vectorize", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
        "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
