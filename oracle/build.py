"""Compile the oracle (plain C, fp64) into oracle/liboracle.so with gcc.

Test infrastructure only: the library never links or loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile ``src`` unconditionally into ``lib`` and return its path."""
    tmp = lib + f".tmp{os.getpid()}"
    cmd = ["gcc", *CFLAGS, src, "-o", tmp, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
