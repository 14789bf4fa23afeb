"""Build libdbs.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m dynamic_block_sparse_gilbert_amd.build [-v]

Every HIP/C++ source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into dynamic_block_sparse_gilbert_amd/libdbs.so.  The
library is written to a temporary name and renamed, so a process that has
the old library loaded is not disturbed.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdbs.so")
ARCH = "gfx950"

SOURCES = [
    "api.cpp",
    "host/perm.cpp",
    "host/stats.cpp",
    "kernels/reorder.hip",
    "kernels/estimate.hip",
    "kernels/mask.hip",
    "kernels/attn.hip",
    "kernels/attn_bwd.hip",
    "kernels/prune.hip",
    "kernels/pooled.hip",
    "kernels/fp32.hip",
]

# Packed fp32 VALU ops are disabled on purpose: only plain fp32 ops are emitted.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# Per-source extra flags.  The attention and estimator kernels are compiled
# without NaN semantics: their maximum reductions then map onto v_max3_f32
# with no canonicalising v_max_f32 x, x in front of every operand.
# Infinities keep their meaning (masked keys are -inf); NaN inputs give an
# undefined result (an exact softmax of them is NaN anyway).
SOURCE_FLAGS = {"kernels/attn.hip": ["-fno-honor-nans"], "kernels/estimate.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []),
           "-x", "hip", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# ---- host-sanitizer build (CPU tests only) -------------------------------------------------
# The host-side sources (argument checks, permutations, the normal quantile) are
# compiled again with AddressSanitizer and UndefinedBehaviorSanitizer on the host
# pass only (the device code is not instrumented) and linked with the ordinary
# kernel objects into _build/asan/libdbs_asan.so.  Python loads it through
# DBS_LIB_PATH with the sanitizer runtime preloaded (see asan_runtime()).
HOST_SOURCES = ["api.cpp", "host/perm.cpp", "host/stats.cpp"]
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_LIB = os.path.join(BUILD, "asan", "libdbs_asan.so")


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload into Python), or ""."""
    root = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib", "clang")
    if not os.path.isdir(root):
        return ""
    for ver in sorted(os.listdir(root), reverse=True):
        p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return ""


def build_host_sanitized(verbose: bool = False) -> str:
    kernel_objs = [os.path.join(BUILD, s.replace("/", "_") + ".o") for s in SOURCES if s not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in kernel_objs):
        build(verbose)
    out = os.path.join(BUILD, "asan")
    os.makedirs(out, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(out, src.replace("/", "_") + ".o")
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-c",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, *DEVICE_FLAGS, *SAN_FLAGS,
               "-x", "hip", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer compile failed: {src}\n{r.stderr}")
        objs.append(obj)
    tmp = SAN_LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libasan", *objs,
           *kernel_objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer link failed\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
