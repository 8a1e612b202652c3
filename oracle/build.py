"""Build the fp64 CPU oracle library (test infrastructure only).

Compiles ``q4_oracle.c`` with gcc into ``libq4oracle.so`` beside it.  No
fast-math and no FP contraction, so every operation rounds as written.
Beside the library it writes ``libq4oracle.so.sha256``, a digest of the
source it was built from, which the loader compares with the source in the
tree.
"""
import hashlib
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4_oracle.c")
LIB = os.path.join(HERE, "libq4oracle.so")
TREE_LIB = LIB  # the in-tree library, whose stamp the loader checks


def source_digest() -> str:
    with open(SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def stamp_path(lib: str) -> str:
    return lib + ".sha256"


def stale_reason(lib: str):
    """None if the library's stamp matches q4_oracle.c, else why not."""
    try:
        with open(stamp_path(lib)) as f:
            stamp = f.read().strip()
    except OSError:
        return "it has no source stamp"
    if stamp != source_digest():
        return "it was built from another q4_oracle.c"
    return None


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-shared", "-fPIC", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    digest = source_digest()
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    with open(stamp_path(LIB), "w") as f:
        f.write(digest + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
