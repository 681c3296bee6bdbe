"""Compile the CPU oracle (test infrastructure) into oracle/libw8a8_oracle.so.

Plain gcc, no fast-math, no FMA contraction, so every rounding the oracle
names happens exactly once.  Usable as a script or through build_oracle().
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "w8a8_oracle.c")
LIB = os.path.join(HERE, "libw8a8_oracle.so")


def build_oracle(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose="-v" in sys.argv))
