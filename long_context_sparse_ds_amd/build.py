"""Build the HIP library libdsparse.so in-tree for gfx950.

    python -m long_context_sparse_ds_amd.build

Every HIP source is compiled with hipcc for gfx950 only; the CPU calibration
file with g++.  Packed-fp32 instruction selection is disabled for all device
code, and kernel arguments are preloaded into SGPRs where supported.  Objects go to long_context_sparse_ds_amd/_build/, the shared library
next to this file.

    python -m long_context_sparse_ds_amd.build --sanitize-host

builds libdsparse_hostsan.so under _build/: the host code of the boundary
(argument checks, workspace planning, launch set-up in ds_api.hip, and the CPU
calibration) instrumented with AddressSanitizer and UndefinedBehaviorSanitizer,
linked with the ordinary kernel objects.  Device code is never instrumented.
Load it with clang's ASan runtime preloaded and DSPARSE_LIB pointing at it.

    python -m long_context_sparse_ds_amd.build --stamps

builds libdsparse_stamps.so beside the library: every kernel source compiled with
DS_STAMPS, so the score, bucket, fused and first-stage kernels record clock
stamps at their phase boundaries (csrc/stamps.h); python -m
long_context_sparse_ds_amd.stamps runs a workload through it and prints the
per-phase timeline.  The ordinary library is built without them.
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
LIB_HOSTSAN = os.path.join(BUILD, "libdsparse_hostsan.so")
LIB_STAMPS = os.path.join(PKG, "libdsparse_stamps.so")

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


# Sanitizers for the host pass only (each flag after -Xarch_host), so no device code is instrumented.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
CXX_SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _llvm_clangxx() -> str:
    for cand in ("/opt/rocm/llvm/bin/clang++", shutil.which("amdclang++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("clang++ of the ROCm toolchain not found")


def asan_runtime() -> str:
    """Path of the shared ASan runtime (with UBSan) of the toolchain that builds the sanitized library."""
    out = subprocess.run([_llvm_clangxx(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if not out or not os.path.exists(out):
        raise RuntimeError("libclang_rt.asan-x86_64.so not found")
    return out


def _objects_current() -> bool:
    """Whether build()'s objects exist and are newer than every source and header."""
    objs = [os.path.join(BUILD, src.replace(".hip", ".o")) for src in HIP_SOURCES]
    if not all(os.path.exists(o) for o in objs):
        return False
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    return min(os.path.getmtime(o) for o in objs) >= max(os.path.getmtime(f) for f in srcs)


def build_host_sanitized(verbose: bool = False) -> str:
    """The library with its host boundary code under ASan + UBSan (kernel objects from build(), rebuilt first
    if they are missing or older than the sources)."""
    if not _objects_current():
        build(verbose)
    san = os.path.join(BUILD, "hostsan")
    os.makedirs(san, exist_ok=True)
    api = os.path.join(san, "ds_api.o")
    cal = os.path.join(san, "calibrate.o")
    flags = [f for f in hip_flags() if f != "-O3"] + ["-O1", "-g"]
    _run([_hipcc(), "-x", "hip", "-c", *flags, *HOST_SANITIZE, os.path.join(CSRC, "ds_api.hip"), "-o", api], verbose)
    _run([_llvm_clangxx(), "-O1", "-g", "-std=c++17", "-fPIC", *CXX_SANITIZE, f"-I{INCLUDE}", "-c",
          os.path.join(CSRC, "calibrate.cpp"), "-o", cal], verbose)
    kernels = [os.path.join(BUILD, src.replace(".hip", ".o")) for src in HIP_SOURCES if src != "ds_api.hip"]
    tmp = LIB_HOSTSAN + ".tmp"
    _run([_hipcc(), "-shared", f"--offload-arch={ARCH}", "-shared-libsan", *HOST_SANITIZE, "-o", tmp, api, cal,
          *kernels], verbose)
    os.replace(tmp, LIB_HOSTSAN)
    return LIB_HOSTSAN


def build_stamped(verbose: bool = False) -> str:
    """The library with the kernels' clock stamps compiled in (-DDS_STAMPS), beside libdsparse.so."""
    out = os.path.join(BUILD, "stamps")
    os.makedirs(out, exist_ok=True)
    hipcc = _hipcc()
    jobs, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(out, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([hipcc, "-x", "hip", "-c", *hip_flags(), "-DDS_STAMPS", os.path.join(CSRC, src), "-o", obj])
    for src in CPP_SOURCES:
        obj = os.path.join(out, src.replace(".cpp", ".o"))
        objs.append(obj)
        jobs.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB_STAMPS + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_STAMPS)
    return LIB_STAMPS


if __name__ == "__main__":
    if "--sanitize-host" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    elif "--stamps" in sys.argv:
        print(build_stamped(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
