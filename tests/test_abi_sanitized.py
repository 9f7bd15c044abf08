"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

api.cpp is compiled with the host C++ compiler together with stand-ins for the
kernel launchers (tests/asan/stub_launch.cpp, which only count calls) and a
driver (tests/asan/abi_driver.cpp) that takes every entry point of
include/hifa4.h through its validation paths and one valid call each: the
documented status, nothing launched on an error, the error text set on failure
and cleared on success.  The sanitizers catch out-of-bounds or invalid memory
use and undefined behaviour in the host code on the way; no GPU code is built.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_c_abi_validation_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "bit_flashattention_hifa4_amd", "csrc"),
           os.path.join(ROOT, "bit_flashattention_hifa4_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "asan", "stub_launch.cpp"),
           os.path.join(ROOT, "tests", "asan", "abi_driver.cpp"), "-o", str(exe)]
    subprocess.check_call(cmd)
    # verify_asan_link_order=0: the environment may preload a library of its own
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr
