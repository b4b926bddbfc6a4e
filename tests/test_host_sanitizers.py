"""The C ABI's host-side validation (csrc/dion_api.cpp with csrc/dion_plan.h) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The API source is built with g++ together with tests/host_san/stubs.cpp (test-only stand-ins for
the device entry points) and tests/host_san/abi_rejects.cpp, which calls every entry point with
the rejection cases of tests/test_abi.py and a few accepted calls, using fake device addresses
that the host must never dereference.  The run must print no sanitizer report and exit 0.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_orthonormalized_optimizer_amd", "csrc")


def test_abi_validation_is_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "abi_rejects")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "dion_api.cpp"),
           os.path.join(ROOT, "tests", "host_san", "stubs.cpp"),
           os.path.join(ROOT, "tests", "host_san", "abi_rejects.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=240)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-3000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert "all cases as expected" in out
