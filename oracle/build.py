"""Build step for the CPU oracle (test infrastructure only).

Compiles oracle.c with the system C compiler into oracle/liboracle.so.
Plain -O2, no fast-math, no FMA contraction, so every binary64 operation
in the oracle is the single correctly rounded IEEE operation it reads as.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-o", LIB + ".tmp", SRC, "-lpthread", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
