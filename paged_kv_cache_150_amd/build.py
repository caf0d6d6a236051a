"""Build libpa.so (the HIP kernels and their C ABI) in-tree for gfx950.

Usage: ``python -m paged_kv_cache_150_amd.build`` or ``build_library()``.
Every call recompiles; objects go to ``paged_kv_cache_150_amd/_build/``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
SOURCES = ["paged_decode.hip", "multi_query.hip", "cache_ops.hip", "measure.hip", "block_pool.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # Keep the compiler from forming packed FP32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [hipcc(), *COMPILE_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build_library(extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every HIP source and link ``libpa.so``; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags or [])
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


# Host-code sanitizers: the host side of every source (argument checks, the
# block pool, launch set-up) built with AddressSanitizer and
# UndefinedBehaviorSanitizer; device code is built as usual. The library
# needs the shared ASan runtime preloaded into the process that loads it
# (asan_runtime()).
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libpa_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-shared-libasan", "-g"]


def asan_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of hipcc's clang."""
    import glob
    root = os.path.dirname(os.path.dirname(hipcc()))
    for cand in sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                              "libclang_rt.asan-x86_64.so"))):
        return cand
    raise RuntimeError("libclang_rt.asan-x86_64.so not found next to hipcc")


def build_sanitized(verbose: bool = False) -> str:
    """Compile every source with host sanitizers into _build_san/libpa_san.so."""
    os.makedirs(SAN_BUILD, exist_ok=True)

    def one(src):
        obj = os.path.join(SAN_BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = [hipcc(), *COMPILE_FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        return obj
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    # The runtime is not linked in: its symbols resolve at load time from the
    # preloaded shared ASan runtime (which carries the UBSan handlers too).
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", SAN_LIB + ".tmp", *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}", file=sys.stderr)
    return SAN_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "sanitized":
        build_sanitized(verbose=True)
    else:
        build_library(verbose=True)
