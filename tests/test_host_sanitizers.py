"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The work partitioners and the C ABI's host paths (validation, planning, plan
inspection) are compiled with g++ -fsanitize=address,undefined together with
a driver that runs them over seeded random ragged batches and invalid inputs
(tests/host/sanitize_driver.cpp; the kernel launchers are stubbed, no HIP
call is reached). The oracle (test infrastructure) gets the same treatment
with gcc (tests/host/oracle_sanitize_driver.c). Any report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "mla_ragged_chunked_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
       "-fno-sanitize-recover=undefined"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def _run(cmd, exe, tmp_path):
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_planner_and_abi_host_paths_under_sanitizers(tmp_path):
    _need("g++")
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("HIP headers not available")
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + CSRC, os.path.join(HOST, "sanitize_driver.cpp"),
           os.path.join(CSRC, "planner.cpp"), os.path.join(CSRC, "abi.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    out = _run(cmd, exe, tmp_path)
    assert "checks passed" in out


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", *SAN, os.path.join(HOST, "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe]
    out = _run(cmd, exe, tmp_path)
    assert "returned 0" in out
