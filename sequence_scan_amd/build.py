"""Build libssmscan.so (gfx950) in-tree with hipcc.

The library is the whole product path: HIP kernels plus the C-ABI host layer.
Flags: packed-FP32 VALU instructions are disabled (the code is written for
scalar fp32 VALU), and floating-point contraction is off so that every fused
multiply-add in the kernels is one written out explicitly (results then do
not depend on how the compiler schedules a template instance).

Machine sinking is disabled: with ROCm 7.2's compiler the MachineSink pass
moved the LDS reads of a tile's recurrence past the workgroup barrier that
ends it (into a successor block created by a later uniform branch), so fast
waves overwrote tile inputs that slow waves had not read yet.  The IR and the
post-isel machine code had the correct order.  tests/test_codegen.py checks
the generated assembly for that symptom (two barriers with no work between).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "api.cpp")]
HEADERS = [os.path.join(CSRC, "internal.h"), os.path.join(os.path.dirname(HERE), "include", "ssmscan.h")]
LIB = os.path.join(HERE, "libssmscan.so")
ARCH = os.environ.get("SSM_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-mllvm", "-disable-machine-sink", "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    """Compile unconditionally; returns the path of libssmscan.so."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["hipcc", *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    noise = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, LIB)
    return LIB


def asm(out_path: str) -> str:
    """Write the gfx950 assembly of the kernels (for inspection)."""
    cmd = ["hipcc", *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-S",
           SOURCES[0], "-o", out_path]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
