"""Compile the CPU oracle (``bsa_oracle.c``) into ``oracle/liboracle.so``.

Test infrastructure only.  Strict IEEE build: no fast-math, no implicit
contraction of multiply-add (the fp32 scoring contract relies on that).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bsa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
        "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
        "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
