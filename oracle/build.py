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
# AddressSanitizer + UBSan build of the same source, for the host-sanitizer
# test (loaded with gcc's libasan preloaded; never by the regular tests)
LIB_SANITIZED = os.path.join(HERE, "liboracle_sanitized.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    # Plain portable flags: no -march (the library is built here and may run on
    # another host), no fast-math, no FMA contraction.
    out = LIB_SANITIZED if sanitize else LIB
    san = (["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"] if sanitize else [])
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-Wall", "-Wextra"] + san + ["-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
