"""Build the gfx950 HIP library ``libq4linear.so`` in-tree.

Every source under ``csrc/`` is compiled with hipcc for gfx950 only, in
parallel, then linked into one shared library beside this file.  No
fast-math flags: fp32 denormals are kept and every operation rounds as IEEE
specifies.  Packed fp32 instructions are disabled for the device code.

Beside the library the build writes ``libq4linear.so.sha256``: a digest of
the sources it was built from (comments and blank space removed), which the
binding compares with the sources in the tree before it loads the library.
"""
import concurrent.futures as cf
import glob
import hashlib
import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libq4linear.so")
TREE_LIB = LIB  # the in-tree library, whose stamp the binding checks
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def source_digest() -> str:
    """sha256 over the HIP sources and the C header with comments and blank
    space removed: edits to comments alone keep it."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*"))) + [os.path.join(INCLUDE, "q4linear.h")]
    for f in files:
        with open(f) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(os.path.basename(f).encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def stamp_path(lib: str) -> str:
    return lib + ".sha256"


def stale_reason(lib: str):
    """None if the library's stamp matches the sources in the tree, else why
    it does not."""
    try:
        with open(stamp_path(lib)) as f:
            stamp = f.read().strip()
    except OSError:
        return "it has no source stamp (built by an older build script?)"
    if stamp != source_digest():
        return "it was built from other sources than those in the tree"
    return None


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device feature flag; that note is noise
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    digest = source_digest()
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    with open(stamp_path(LIB), "w") as f:
        f.write(digest + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
