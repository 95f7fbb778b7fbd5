"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds tests/host/host_checks.cpp together with the library's C-ABI layer
(csrc/api.cpp) with g++ -fsanitize=address,undefined and runs it: argument
validation, the hand-off to the launchers (with stand-ins for the HIP
runtime and the kernels), the host block split helpers and the kernel
selection rules of csrc/plan.hpp.  No GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


def test_host_checks_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("g++ or the HIP headers are missing")
    exe = tmp_path / "host_checks"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
           os.path.join(ROOT, "block_quantized_decode_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "host", "host_checks.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host checks passed" in run.stdout
