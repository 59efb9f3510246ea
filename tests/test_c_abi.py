"""The C ABI from plain C: tests/c_abi/abi_check.c is compiled with gcc as C11 against
include/moe.h, linked to the in-tree libmoe_hip.so and run. It needs no GPU (every call
it makes returns before any HIP call)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_mixture_experts_sum_amd")
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_check.c")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def lib():
    path = os.path.join(PKG, "libmoe_hip.so")
    if not os.path.exists(path):
        from sparse_mixture_experts_sum_amd import build
        build.build()
    return path


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs gcc and the ROCm headers")
def test_c_program_against_the_header(lib, tmp_path):
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"), SRC, "-o", str(exe),
           "-L", PKG, "-lmoe_hip", f"-Wl,-rpath,{PKG}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "passed: 0 failure(s)" in r.stdout
