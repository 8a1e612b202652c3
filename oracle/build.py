"""Build the fp64 CPU oracle library (test infrastructure only).

Compiles ``q4_oracle.c`` with gcc into ``libq4oracle.so`` beside it.  No
fast-math and no FP contraction, so every operation rounds as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4_oracle.c")
LIB = os.path.join(HERE, "libq4oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-shared", "-fPIC", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
