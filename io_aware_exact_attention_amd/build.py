"""Compile the HIP kernels and the C-ABI host layer into ``libmiattn.so`` (in-tree).

gfx950 only.  Packed-fp32 VALU instructions are switched off for the device code.  Each
source is compiled to an object under ``_build/`` (in parallel), then linked.

``build_sanitized_library()`` links a second copy for CPU-side checking: the host layer
(miattn_api.cpp: validation, planning, parameter set-up) compiled with AddressSanitizer
and UndefinedBehaviorSanitizer, the kernel objects unchanged.  It is loaded only by the
sanitizer test, through MIATTN_LIB, with the ASan runtime preloaded.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libmiattn.so")
OBJ_DIR = os.path.join(REPO_DIR, "_build")
SAN_LIB_PATH = os.path.join(OBJ_DIR, "libmiattn_san.so")

KERNEL_SOURCES = [
    "csrc/prefill_gfx950.hip",
    "csrc/decode_gfx950.hip",
    "csrc/backward_gfx950.hip",
]
HOST_SOURCE = "csrc/miattn_api.cpp"
SOURCES = KERNEL_SOURCES + [HOST_SOURCE]
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# host-side sanitizers only (each flag applies to the host compilation alone)
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def _object(src: str, tag: str = "") -> str:
    base = os.path.splitext(os.path.basename(src))[0]
    return os.path.join(OBJ_DIR, base + tag + ".o")


def _compile(src: str, extra=(), tag: str = "") -> str:
    obj = _object(src, tag)
    _run([hipcc_path(), *FLAGS, *extra, "-I", os.path.join(REPO_DIR, "include"), "-c",
          os.path.join(PKG_DIR, src), "-o", obj])
    return obj


def build_library(verbose: bool = False) -> str:
    """Build libmiattn.so next to this file; returns its path.  Always recompiles."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc_path(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    _run(cmd)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (to preload into a host process)."""
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc_path())))
    cands = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not cands:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found next to hipcc")
    return cands[-1]


def build_sanitized_library() -> str:
    """Link _build/libmiattn_san.so: the kernel objects of the last build_library() (built
    now if missing) and the host layer compiled with ASan and UBSan."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [_object(s) for s in KERNEL_SOURCES]
    missing = [s for s, o in zip(KERNEL_SOURCES, objs) if not os.path.exists(o)]
    if missing:
        with ThreadPoolExecutor(len(missing)) as ex:
            list(ex.map(_compile, missing))
    host = _compile(HOST_SOURCE, SAN_FLAGS, tag="_san")
    tmp = SAN_LIB_PATH + ".tmp"
    _run([hipcc_path(), "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          *objs, host, "-o", tmp])
    os.replace(tmp, SAN_LIB_PATH)
    return SAN_LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
