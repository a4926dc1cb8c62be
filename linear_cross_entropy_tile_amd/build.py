"""Builds libflce.so, the HIP library behind include/flce.h, in-tree for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libflce.so")
SOURCES = [os.path.join(PKG, "csrc", "flce_api.hip")]
HEADERS = [os.path.join(ROOT, "include", "flce.h"),
           os.path.join(PKG, "csrc", "flce_layout.hpp"),
           os.path.join(PKG, "csrc", "flce_plan.hpp"),
           os.path.join(PKG, "csrc", "flce_gemm.hpp"),
           os.path.join(PKG, "csrc", "flce_kernels.hpp")]

# Packed fp32 VALU forms are switched off for all device code.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I" + os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compiles the library (always) and returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "flce_c_check.c")
C_CHECK = os.path.join(ROOT, "tests", "c_abi", "flce_c_check")


def build_c_check(verbose: bool = False) -> str:
    """Compiles the plain-C99 program that drives the C ABI (a GPU test runs
    it) against the in-tree library, with gcc: the header must be valid C."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(rocm, "include"),
           C_CHECK_SRC, "-o", C_CHECK + ".tmp", "-L" + PKG, "-lflce",
           "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../linear_cross_entropy_tile_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("gcc failed:\n" + res.stdout + res.stderr)
    os.replace(C_CHECK + ".tmp", C_CHECK)
    return C_CHECK


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_check(verbose=True))
