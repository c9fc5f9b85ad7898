"""Build the HIP library libzs.so in-tree for gfx950 with hipcc.

Usage: python -m zero_sharded_mixed_buffer_amd.build   (or build() from Python)
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzs.so")

SOURCES = ["zs_abi.cpp", "zs_kernels.hip", "zs_probe.hip"]
HOST_SOURCES = ["zs_host.cpp", "zs_plan.cpp"]  # plain C++ (host step, planner), built by the host compiler
HEADERS = ["zs_internal.h", "zs_host.h", "zs_plan.h"]

# Packed fp32 vector ops are disabled for all device code; fp contraction is left to the
# sources, which switch it off where an fp64 expression must round like its plain form.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# The host step must round like its plain form (no fused multiply-add); math errno is off so
# that sqrt can be vectorised (IEEE results are unchanged).
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off", "-fno-math-errno", "-pthread"]


# roctx ranges around the entry points (profiler markers).
LINK_LIBS = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]


def cxx() -> str:
    return os.environ.get("CXX", "g++")


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    """Compile every source and link libzs.so next to this file; returns its path."""
    objs = []
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        _run([cxx(), *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs, *LINK_LIBS], verbose)
    os.replace(tmp, LIB)
    build_c_consumer(verbose)
    return LIB


# A plain C++ program that drives the library through zs.h and the HIP runtime only, with
# no Python (tests/test_gpu_c_abi.py runs it); host code, so the host compiler builds it.
C_CONSUMER_SRC = os.path.join(ROOT, "tests", "c", "abi_gpu.cpp")
C_CONSUMER = os.path.join(ROOT, "tests", "c", "abi_gpu")


def build_c_consumer(verbose: bool = False) -> str:
    tmp = C_CONSUMER + ".tmp"
    _run([cxx(), "-O2", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", INCLUDE,
          C_CONSUMER_SRC, "-o", tmp, "-L", PKG, "-lzs", "-Wl,-rpath,$ORIGIN/../../zero_sharded_mixed_buffer_amd",
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], verbose)
    os.replace(tmp, C_CONSUMER)
    return C_CONSUMER


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout)
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}")
    if verbose and res.stdout.strip():
        print(res.stdout)


if __name__ == "__main__":
    print(build(verbose=True))
