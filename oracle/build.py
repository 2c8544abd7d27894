"""Compile the oracle's C loops (oracle/gemv.c) into oracle/_gemv.so with gcc.

TEST INFRASTRUCTURE ONLY."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemv.c")
LIB = os.path.join(HERE, "_gemv.so")


def build(verbose: bool = True) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build()
