"""Build libqmoe.so (HIP C++ for gfx950) in-tree with hipcc.

Usage: python -m block_quantized_moe_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqmoe.so")
ARCH = "gfx950"

HIP_SOURCES = ["dequant.hip", "plan.hip", "gemm.hip", "gemv.hip", "combine.hip", "router.hip", "api.hip"]
HOST_SOURCES = ["split.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]
# Packed fp32 arithmetic stays off (the compiler forms it from plain float code).
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        o = os.path.join(OBJ, src + ".o")
        jobs.append([cc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", o])
    for src in HOST_SOURCES:
        o = os.path.join(OBJ, src + ".o")
        jobs.append([cc, *COMMON, "-x", "c++", "-c", os.path.join(CSRC, src), "-o", o])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
