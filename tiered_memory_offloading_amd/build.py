"""Build libdak.so (the C-ABI library of the split operators) for gfx950, in-tree.

HIP sources are compiled with hipcc for gfx950 only; the pure C++ sources
(planner, error state) with g++.  Every translation unit uses
-ffp-contract=off so floating-point expressions are evaluated exactly as
written (the planner's plans and the kernels' reduction orders depend on it),
and HIP code is built without packed-fp32 instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdak.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIP_SOURCES = ["runtime.hip", "splitk_gemm.hip", "splitk_gemm_staged.hip", "splitk_gemm_tiled.hip", "splitk_gemm_fp8.hip",
               "split_attn.hip", "probe.hip"]
CXX_SOURCES = ["errors.cpp", "planner.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", "-ffp-contract=off", "-Wall", f"-I{INCLUDE}"]
HIP_FLAGS = COMMON + [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libdak.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cmds = []
    objs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    for s in CXX_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append([CXX] + COMMON + ["-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    out = _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
