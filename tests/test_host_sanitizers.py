"""Host code under the address and undefined-behaviour sanitizers (CPU only).

Two programs are built with gcc/g++ and ``-fsanitize=address,undefined``:
``tests/sanitize/oracle_driver.c`` runs every function of the fp64 oracle on
small seeded inputs (finite results, decode steps equal to the forward, results
independent of the thread count, bad arguments refused), and
``tests/sanitize/abi_driver.cpp`` drives the C ABI's host layer
(``gdr_abi.cpp``: descriptor checks, workspace sizing and carving, aliasing and
alignment checks, the cut of the state passes into ranges) with the kernel
launchers replaced by host stand-ins that check every carved workspace pointer
and chunk range.  Any sanitizer report aborts the program and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", *SAN, os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "gdr_oracle.c"), "-lm", "-pthread", "-o", exe])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"))
    assert "0 failures" in r.stdout


def test_abi_host_layer_under_sanitizers(tmp_path):
    if not shutil.which("g++") or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers not available")
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "gated_delta_rule_37_amd", "csrc")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "abi_stubs.cpp"),
          os.path.join(csrc, "gdr_abi.cpp"), os.path.join(csrc, "gdr_prof.cpp"),
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    # the HIP runtime keeps allocations until exit, which the leak checker
    # would report; leaks of this program's own code are not the subject here
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", HIP_VISIBLE_DEVICES=""))
    assert "0 failures" in r.stdout
