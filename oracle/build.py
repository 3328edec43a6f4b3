"""Build the CPU oracle (oracle.c -> liboracle.so) with gcc.

Test infrastructure: the oracle is compiled so that tests, the smoke check
and the benchmark's CPU-baseline leg can call it.  The flags keep binary32
arithmetic exactly as written: no FMA contraction, no fast-math, no
flush-to-zero, scalar code.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-fno-tree-vectorize", "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    """Compile the oracle library; returns its path."""
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
