"""Build the CPU oracle (``oracle.c``) into ``liboracle.so`` with gcc.

Test infrastructure: the product library never builds, loads or calls this.

Flags: ``-ffp-contract=off`` so no multiply-add is fused (GCC's GNU-mode
default is ``fast``), no ``-ffast-math`` (keeps IEEE division, sqrt and
subnormals), no ``-march=native`` (keeps x86-64 SSE2 binary32 arithmetic,
where every float operation rounds once to binary32).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-O2",
    "-std=c11",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wextra",
    "-Werror",
]


def build_oracle(verbose: bool = False) -> str:
    """Compile the oracle; returns the path of the shared library."""
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SOURCE, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build_oracle(verbose="-v" in sys.argv))
