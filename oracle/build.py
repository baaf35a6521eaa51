"""Build the CPU oracle library (test infrastructure only).

Plain gcc, fp64 arithmetic, no FMA contraction, OpenMP over tokens in the
row-independent operation.  Writes oracle/liborc.so next to this file.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rrp_oracle.c")
LIB = os.path.join(HERE, "liborc.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
        "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
