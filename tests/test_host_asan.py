"""The host library code (kda_api.cpp: argument checks, overlap checks, error messages, status
strings, size queries) built with g++ and AddressSanitizer + UndefinedBehaviorSanitizer, and run
through the C ABI on rejected arguments (CPU test: the kernel launchers are host-only stand-ins
in tests/host_asan/stubs.cpp, so no device code is built or run)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "delta_rule_recurrent_kda_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_asan")


def test_api_checks_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / "kda_host_asan")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", os.path.join(CSRC, "kda_api.cpp"),
           os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp"), "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("KDA_VALIDATE", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "done, 0 failures" in r.stdout, r.stdout[-4000:] + r.stderr[-4000:]
