"""Builds libxattn.so for gfx950 in-tree: HIP kernels with hipcc, host code with g++.

Usage: python -m ragged_attention_serving_amd.build [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libxattn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

ARCH = "gfx950"
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    # no packed fp32 instructions (v_pk_*_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{CSRC}", f"-I{INCLUDE}",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
             f"-I{ROCM}/include", f"-I{CSRC}", f"-I{INCLUDE}"]

HIP_SOURCES = ["attn_f32.hip", "attn_decode.hip", "attn_mma.hip", "merge.hip", "write_kv.hip", "scratch.hip"]
CXX_SOURCES = ["partition.cpp", "api.cpp"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if err.strip():
            print(err, flush=True)


def build(verbose: bool = False) -> str:
    """Compiles every source and links libxattn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    cxx = shutil.which("g++") or "g++"
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    # -z defs: a symbol left undefined (a kernel whose launch stub a compilation pass did
    # not emit, say) fails the link here instead of the library's first load
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-Wl,-z,defs"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
