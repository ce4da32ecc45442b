"""Builds libhswa.so (HIP kernels for gfx950 + host C++) in the package dir.

    python -m hybrid_sliding_window_hswa_amd.build

Kernels are compiled by hipcc for gfx950 only; host-only C++ by g++ against
the HIP runtime headers; the shared library links libamdhip64.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhswa.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["kernels_kv.hip", "kernels_decode.hip", "kernels_prefill.hip"]
CPP_SOURCES = ["pool.cpp", "capi.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
             "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    """Compiles every source and links the library; returns its path."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    cxx = shutil.which("g++") or "c++"
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append((o, [hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, s), "-o", o]))
    for s in CPP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append((o, [cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", o]))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for (o, cmd), out in zip(jobs, outs):
            print(" ".join(cmd))
            if out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
          *[o for o, _ in jobs], f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
