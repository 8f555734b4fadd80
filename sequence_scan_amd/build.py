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
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
# Device translation units, as (source, extra defines, object name).  The
# scan kernel template is instantiated by scan_inst.hip once per (input dtype,
# output dtype, input coefficient): eight units that compile in parallel.
def _scan_units():
    units = []
    for zoh in (0, 1):
        for tin, nin in (("float", "f32"), ("uint16_t", "bf16")):
            for tout, nout in (("float", "f32"), ("uint16_t", "bf16")):
                fn = f"launch_scan_{nin}_{nout}" + ("_zoh" if zoh else "")
                units.append((os.path.join(CSRC, "scan_inst.hip"),
                              [f"-DSSM_INST_TIN={tin}", f"-DSSM_INST_TOUT={tout}", f"-DSSM_INST_ZOH={zoh}",
                               f"-DSSM_INST_FN={fn}"], fn))
    return units


DEVICE_UNITS = _scan_units() + [(os.path.join(CSRC, f), [], f.split(".")[0]) for f in ("scan.hip", "conv.hip", "bwd.hip", "ssd.hip")]
HOST_UNITS = [(os.path.join(CSRC, "api.cpp"), [], "api")]
SOURCES = sorted({u[0] for u in DEVICE_UNITS + HOST_UNITS})
HEADERS = [os.path.join(CSRC, f) for f in ("internal.h", "device.h", "scan_kernel.h")] + [
    os.path.join(os.path.dirname(HERE), "include", "ssmscan.h")]
LIB = os.path.join(HERE, "libssmscan.so")
# The benchmark's probes (VALU issue rates, streaming bandwidth): a separate
# small library, not part of the scan library's ABI.
PROBE_SRCS = [os.path.join(CSRC, "valu_probe.hip"), os.path.join(CSRC, "stream_probe.hip")]
PROBE_LIB = os.path.join(HERE, "libssmprobe.so")
ARCH = os.environ.get("SSM_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-mllvm", "-disable-machine-sink", "-Wall", "-Wno-unused-function",
]


def _code_tokens(text: str) -> bytes:
    """The source with its comments removed and each run of whitespace made one
    space: an edit of a comment leaves the code, and so its hash, unchanged.
    String and character literals are kept whole."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split()).encode()


def kernel_source_sha256() -> str:
    """One hash over the code of every device source and header (in a fixed
    order, comments and layout left out): the identity of the kernels that a
    profile was taken of."""
    import hashlib
    h = hashlib.sha256()
    for path in sorted({u[0] for u in DEVICE_UNITS} | set(HEADERS)):
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "r", encoding="utf-8") as f:
            h.update(_code_tokens(f.read()))
    return h.hexdigest()


def _run_all(cmds, verbose):
    """Run the compiler commands in parallel; raise with the output of any failure."""
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    failed = []
    for cmd, p in zip(cmds, procs):
        out, _ = p.communicate()
        # the host pass does not know the packed-fp32 target feature; that warning is expected
        noise = [ln for ln in out.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append(" ".join(cmd) + "\n" + "\n".join(noise))
        elif verbose and noise:
            print("\n".join(noise))
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(failed))


def build(verbose: bool = False) -> str:
    """Compile unconditionally; returns the path of libssmscan.so."""
    tmp = LIB + f".tmp{os.getpid()}"
    with tempfile.TemporaryDirectory(prefix="ssmscan_build_") as od:
        units = DEVICE_UNITS + HOST_UNITS
        objs = [os.path.join(od, name + ".o") for _, _, name in units]
        comp = [f for f in FLAGS if f != "-shared"]
        _run_all([["hipcc", *comp, *defs, "-c", src, "-o", obj] for (src, defs, _), obj in zip(units, objs)], verbose)
        # -z defs: a launcher declared but built in no unit fails here, not at load time
        ptmp = PROBE_LIB + f".tmp{os.getpid()}"
        _run_all([["hipcc", *FLAGS, "-Wl,-z,defs", *objs, "-o", tmp],
                  ["hipcc", *FLAGS, "-Wl,-z,defs", *PROBE_SRCS, "-o", ptmp]], verbose)
    os.replace(tmp, LIB)
    os.replace(ptmp, PROBE_LIB)
    return LIB


def asm(out_path: str) -> str:
    """Write the gfx950 assembly of every device translation unit, concatenated
    (for inspection and the code-generation checks)."""
    with tempfile.TemporaryDirectory(prefix="ssmscan_asm_") as od:
        outs = [os.path.join(od, name + ".s") for _, _, name in DEVICE_UNITS]
        flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
        _run_all([["hipcc", *flags, *defs, "--cuda-device-only", "-S", src, "-o", o]
                  for (src, defs, _), o in zip(DEVICE_UNITS, outs)], False)
        with open(out_path, "w") as f:
            for o in outs:
                with open(o) as g:
                    f.write(g.read())
    return out_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
