"""Compile the CPU oracle (``bsa_oracle.c``) into ``oracle/liboracle.so``.

Test infrastructure only.  Strict IEEE build: no fast-math, no implicit
contraction of multiply-add (the fp32 scoring contract relies on that).

``--sanitize`` builds the same library with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; every UB report aborts).  A
library built that way must be loaded by a process that has the ASan runtime
preloaded, e.g. ``LD_PRELOAD=$(gcc -print-file-name=libasan.so)
ASAN_OPTIONS=detect_leaks=0 python -m pytest tests -m "not gpu" -k oracle``;
rebuild without the flag afterwards.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bsa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
        "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
        *(SANITIZE if sanitize else []),
        "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
