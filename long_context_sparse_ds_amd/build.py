"""Build the HIP library libdsparse.so in-tree for gfx950.

    python -m long_context_sparse_ds_amd.build

Every HIP source is compiled with hipcc for gfx950 only; the CPU calibration
file with g++.  Packed-fp32 instruction selection is disabled for all device
code, and kernel arguments are preloaded into SGPRs where supported.  Objects go to long_context_sparse_ds_amd/_build/, the shared library
next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsparse.so")

HIP_SOURCES = ["ds_api.hip", "pack.hip", "score.hip", "select.hip", "selattn.hip", "bucket.hip", "attn.hip",
               "hip_search.hip"]
CPP_SOURCES = ["calibrate.cpp"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def hip_flags():
    # Kernel arguments: the first 14 dwords are preloaded into SGPRs at wave
    # launch where the firmware supports it (the code keeps a fallback path).
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False) -> str:
    """Compile every source and link libdsparse.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([hipcc, "-x", "hip", "-c", *hip_flags(), os.path.join(CSRC, src), "-o", obj])
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        objs.append(obj)
        jobs.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
