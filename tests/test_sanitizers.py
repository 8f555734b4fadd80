"""The oracle and the C-ABI host layer built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU.

* ``tests/sanitize/oracle_driver.c`` runs every oracle function on small and
  empty inputs, with and without the optional ones, on several threads;
* ``tests/sanitize/abi_driver.cpp`` drives every entry point of
  ``include/ssmscan.h`` through ``api.cpp`` over a host-only stand-in for the HIP
  runtime and the kernel launchers (``tests/sanitize/fake_runtime.cpp``): valid
  calls with buffers of exactly their documented sizes, each launcher stub
  reading both ends of every buffer and workspace region handed to its kernel,
  rejected calls, and a workspace allocation that fails.

Both are plain host builds with g++/gcc (no device code is compiled), so the
sanitizers cover host code only.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
HIP_INCLUDE = "/opt/rocm/include"


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def _build_and_run(cmd, exe, expect):
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if b.returncode != 0 and "asan" in (b.stderr or "").lower() and "cannot find" in b.stderr:
        pytest.skip("the sanitizer runtime is not installed")
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert expect in r.stdout, r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_driver")
    _build_and_run(["gcc", "-std=c11", *SAN, os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(HERE, "sanitize", "oracle_driver.c"), "-lm", "-lpthread", "-o", exe],
                   exe, "oracle driver ok")


def test_host_layer_under_asan_ubsan(tmp_path):
    _need("g++")
    if not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")):
        pytest.skip("HIP headers not found")
    exe = str(tmp_path / "abi_driver")
    _build_and_run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INCLUDE}",
                    os.path.join(ROOT, "sequence_scan_amd", "csrc", "api.cpp"),
                    os.path.join(HERE, "sanitize", "fake_runtime.cpp"),
                    os.path.join(HERE, "sanitize", "abi_driver.cpp"), "-o", exe],
                   exe, "abi driver ok")
