"""Build the HIP library in-tree: ``sparse_mixture_experts_sum_amd/libmoe_hip.so``.

Every ``csrc/*.hip`` file is compiled for gfx950 with hipcc into ``_build/`` and the
objects are linked into one shared library exporting the C ABI of
``include/moe.h``. Run ``python -m sparse_mixture_experts_sum_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_hip.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Werror",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    cmds = []
    for s in srcs:
        o = os.path.join(BUILD, os.path.basename(s)[:-4] + ".o")
        objs.append(o)
        cmds.append([HIPCC, *CFLAGS, "-c", s, "-o", o])
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(cmds))) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc != 0:
            if out.strip():
                print(out, file=sys.stderr)
        if rc != 0:
            failed = True
            print(f"FAILED: {' '.join(cmd)}", file=sys.stderr)
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
