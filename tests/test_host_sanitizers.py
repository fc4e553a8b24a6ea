"""CPU test: the C ABI's host code (api.cpp) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, with the HIP runtime calls
and kernel launchers replaced by host stubs (tests/host/stubs.cpp), driven
through every plan shape class and validation path (tests/host/driver.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structured_state_space_dplr_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "driver")
    sanitize = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
    cmd = ["g++", "-std=c++17", "-O1", "-g", *sanitize, "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
           os.path.join(CSRC, "api.cpp"), os.path.join(HOST, "stubs.cpp"),
           os.path.join(HOST, "driver.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "ok" in run.stdout
