"""Compile the CPU oracle (oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is a checker, never part of the product
path.  Plain IEEE arithmetic: no fast-math, no FMA contraction, so the fp64
sums keep the order the source states.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose=False):
    cmd = ["gcc", "-O3", "-std=c99", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-fPIC", "-shared", "-Wall", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
