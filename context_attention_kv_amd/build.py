"""Build libcakv.so in-tree with hipcc for gfx950.

    python -m context_attention_kv_amd.build

Compiles every source under csrc/ (HIP kernels and the C ABI host code) into
one shared library next to this file. No torch extension machinery: the
library has a plain C ABI (include/cakv.h) and is loaded with ctypes.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcakv.so")
SOURCES = ["api.cpp", "fwd_bf16.hip", "fwd_f32.hip", "state_ops.hip", "diag_mfma.hip", "decode_bf16.hip", "bwd_bf16.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcakv)")


def flags() -> list:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # keep the compiler from forming packed fp32 ALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
        "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link libcakv.so; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, *flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    # roctx: the named ranges the C ABI layer pushes around its calls
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
