"""Build the CPU oracle shared library (oracle/liboracle.so) with gcc.

TEST INFRASTRUCTURE ONLY: the oracle is the correctness reference for the
GPU library and is loaded by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # Plain portable flags: no -march (the library is built here and may run on
    # another host), no fast-math, no FMA contraction.
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
