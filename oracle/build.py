"""Compile the C oracle into oracle/libmoe_oracle.so with gcc.

Test infrastructure: the oracle is the checker, never part of the product.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(verbose=False):
    """Always recompile (plain -O2, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
