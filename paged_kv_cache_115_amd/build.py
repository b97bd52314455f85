"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python paged_kv_cache_115_amd/build.py        # or __graft_entry__.build()

Every translation unit is compiled with packed-FP32 instruction selection
disabled (hipcc host passes warn that they do not know the feature; the
warning is harmless).  Objects go to _build/, the library next to this file.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")

ARCH = os.environ.get("PAGEDKV_ARCH", "gfx950")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
SOURCES = ["abi.cpp", "block_manager.cpp", "validate.cpp", "step.cpp", "cache_kernels.hip", "decode_kernels.hip", "decode_f32_kernels.hip", "noalloc.hip",
           "probe_kernels.hip"]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libpagedkv.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-only library for the address and undefined-behaviour sanitizers: the
# host sources (C ABI checks, block manager, planner, validation, step
# preparation) built with g++ and -fsanitize, the kernel launchers replaced by
# host_stubs.cpp.  A CPU-only target: it has no kernels, every GPU entry point
# runs its host checks and then fails.  Used by tests/test_sanitized_host.py.
HOST_SOURCES = ["abi.cpp", "block_manager.cpp", "validate.cpp", "step.cpp", "host_stubs.cpp"]
SANITIZED_LIB = os.path.join(BUILD, "sanitize", "libpagedkv_host_sanitized.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build_host_sanitized(verbose: bool = False) -> str:
    """Compile the host sources with g++ under ASan and UBSan; returns the
    library path."""
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found: the sanitized host library cannot be built")
    os.makedirs(os.path.dirname(SANITIZED_LIB), exist_ok=True)
    cmd = [gxx, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", *SANITIZE_FLAGS, "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", INCLUDE, "-I", CSRC, *[os.path.join(CSRC, f) for f in HOST_SOURCES],
           "-L", "/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", SANITIZED_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed on the sanitized host build:\n{res.stderr}")
    os.replace(SANITIZED_LIB + ".tmp", SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
