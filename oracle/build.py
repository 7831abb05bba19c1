"""Build the CPU oracle shared library (test infrastructure only).

gcc, -O2, no fast-math, no FMA contraction: every float operation in the
oracle is one binary32 round-to-nearest-even operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "jas_oracle.c")
LIB = os.path.join(HERE, "libjas_oracle.so")

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-pthread", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
