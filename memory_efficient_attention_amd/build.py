"""Build the HIP library ``libmea.so`` in-tree with hipcc for gfx950.

Usage: ``python -m memory_efficient_attention_amd.build`` (or ``build()``).
The library lands next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_PATH = os.path.join(PKG_DIR, "libmea.so")
SOURCES = ["fwd_prefill.hip", "fwd_decode.hip", "bwd.hip", "ffn.hip", "mea_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def compile_flags():
    return [
        "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC,
        # no packed float32 VALU forms in any kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link ``libmea.so``; returns its path."""
    cc = hipcc()
    objs = []
    tmp_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(tmp_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmp_dir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *compile_flags(), *(extra_flags or []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp_lib = LIB_PATH + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
