"""Compiles the C11 test client (xattn_client.c) against include/xattn.h and the built
libxattn.so. The binary goes next to the library's objects and finds the library
through its rpath. Test infrastructure: the library itself never uses it."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "ragged_attention_serving_amd")
SRC = os.path.join(HERE, "xattn_client.c")
OUT = os.path.join(PKG, "_build", "xattn_client")
LIB = os.path.join(PKG, "libxattn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    """Compiles the client if it is missing or older than its source or the library."""
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built")
    if (os.path.exists(OUT) and os.path.getmtime(OUT) >= os.path.getmtime(SRC)
            and os.path.getmtime(OUT) >= os.path.getmtime(LIB)):
        return OUT
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cc = shutil.which("gcc") or "gcc"
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC, "-o", OUT + ".tmp",
           f"-L{PKG}", "-l:libxattn.so", f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/..", f"-Wl,-rpath,{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"client build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(OUT + ".tmp", OUT)
    return OUT
