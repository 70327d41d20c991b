"""Build the HIP library for gfx950: hipcc each source, link one shared object.

Usage: python -m additive_codebook_matmul_amd.build   (or call build_library()).
The library lands next to this file as libaqlm_mi355x.so; objects go under
_build/. Every call recompiles from source. build_host_library() compiles the
separate host GEMV library (libaqlm_host.so, g++ with OpenMP);
build_ceiling_library() the benchmark's measurement kernels
(libaqlm_ceiling.so).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libaqlm_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ("api.hip", "dequant.hip", "gemv.hip", "gemv_mfma.hip", "gemv_slice.hip", "gemm.hip",
           "gemm_mid.hip", "gemm_tile.hip", "general.hip", "encode.hip")
ARCH = "gfx950"
HOST_SOURCE = "host_gemv.cpp"
HOST_LIB_PATH = os.path.join(PKG_DIR, "libaqlm_host.so")
# measurement kernels of the benchmark (read and gather ceilings), a library
# of their own so that the product library exports only its C-ABI
CEILING_SOURCE = "ceiling.hip"
CEILING_LIB_PATH = os.path.join(PKG_DIR, "libaqlm_ceiling.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # no packed fp32 instructions anywhere in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build_library(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


def build_host_library(verbose: bool = True) -> str:
    cxx = os.environ.get("CXX") or shutil.which("g++") or "g++"
    tmp = HOST_LIB_PATH + ".tmp"
    cmd = [cxx, "-O3", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-fvisibility=hidden",
           "-Wall", "-I", INCLUDE, os.path.join(CSRC, HOST_SOURCE), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"host library build failed:\n{res.stderr}")
    os.replace(tmp, HOST_LIB_PATH)
    if verbose:
        print(f"built {HOST_LIB_PATH}", file=sys.stderr)
    return HOST_LIB_PATH


def build_ceiling_library(verbose: bool = True) -> str:
    tmp = CEILING_LIB_PATH + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", os.path.join(CSRC, CEILING_SOURCE), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"ceiling library build failed:\n{res.stderr}")
    os.replace(tmp, CEILING_LIB_PATH)
    if verbose:
        print(f"built {CEILING_LIB_PATH}", file=sys.stderr)
    return CEILING_LIB_PATH


if __name__ == "__main__":
    build_library()
    build_host_library()
    build_ceiling_library()
