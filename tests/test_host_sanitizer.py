"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: csrc/moe_api.hip (argument checks, 64-bit size arithmetic on caller-controlled shapes,
workspace layout, launch sequence, stage timing) is compiled as plain C++ with g++, linked
against host-only stand-ins of the kernel launchers (tests/host_sanitize/stub_kernels.cpp,
which also check that every workspace buffer handed to a launcher fits inside the
workspace), and driven through every error path and a sweep of about 600k extreme shapes
(tests/host_sanitize/host_checks.cpp). No GPU, no HIP compiler: the device kernels are not
compiled for this test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "sparse_mixture_experts_sum_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_checks"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-I", SAN,
           "-x", "c++", os.path.join(CSRC, "moe_api.hip"),
           "-x", "c++", os.path.join(SAN, "stub_kernels.cpp"), os.path.join(SAN, "host_checks.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stdout + r.stderr).lower():
        pytest.skip("the sanitizer runtime is not installed: " + r.stderr[-300:])
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed: 0 failure(s)" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out
