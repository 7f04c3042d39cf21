"""Compile the HIP kernels and the C-ABI host layer into ``libmiattn.so`` (in-tree).

gfx950 only.  Packed-fp32 VALU instructions are switched off for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libmiattn.so")

SOURCES = [
    "csrc/prefill_gfx950.hip",
    "csrc/decode_gfx950.hip",
    "csrc/backward_gfx950.hip",
    "csrc/miattn_api.cpp",
]
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def build_library(verbose: bool = False) -> str:
    """Build libmiattn.so next to this file; returns its path.  Always recompiles."""
    srcs = [os.path.join(PKG_DIR, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc_path(), *FLAGS, "-I", os.path.join(REPO_DIR, "include"), *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
