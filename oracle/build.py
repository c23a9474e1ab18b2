"""Build the CPU oracle shared library (test infrastructure only).

``gcc -O2 -fopenmp``, no fast-math, so that fp32 division and ``rintf`` keep
their IEEE round-to-nearest-even meaning.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zq_oracle.c")
LIB = os.path.join(HERE, "libzq_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
