"""Compile the CPU oracle (plain C, single-threaded) into oracle/liboracle.so.

The flags keep binary32 arithmetic exactly as written: no contraction of a
multiply and an add into a fused multiply-add, no fast-math reassociation.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
          "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
