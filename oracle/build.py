"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, -O2, no FMA contraction, OpenMP over independent rows.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
        "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
        os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
