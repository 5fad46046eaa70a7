"""Build the FP64 CPU oracle library (TEST INFRASTRUCTURE ONLY).

Compiles oracle/kda_oracle.c with gcc into oracle/libkda_oracle.so. FP
contraction is off so every operation is a plain IEEE-754 double operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=gnu11", "-O2", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
        "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
