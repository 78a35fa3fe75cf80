"""Compile the HIP library ``librga.so`` for gfx950 with hipcc.

Loaded by file path (``__graft_entry__.build()``), never through the package,
whose import needs the built library.

Sources: ``csrc/*.hip`` (kernels) and ``csrc/api.cpp`` (C ABI). Each is
compiled to an object in ``_build/`` (in parallel), then linked in-tree next
to this file so the library travels with the source tree.

Flags that carry meaning:
  -ffp-contract=off        no multiply-add contraction (the arithmetic is
                           binary32 multiply, then binary32 add)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                           no packed fp32 instructions
  (no -ffast-math, no -fgpu-flush-denormals-to-zero: IEEE division and
  square root, binary32 subnormals kept)
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

CSRC = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(CSRC)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "librga.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Wall",
    "-Wextra",
    f"-I{INCLUDE}",
]
DEVICE = [
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [
        os.path.join(CSRC, "api.cpp")]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build_library(verbose: bool = False) -> str:
    """Compile and link librga.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
           "-o", tmp, "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
