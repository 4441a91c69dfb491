"""Build libpagedattn.so in-tree for gfx950.

Run ``python -m paged_kv_cache_block_amd.build`` (or ``__graft_entry__.build()``).
Each source compiles to an object in ``_build/`` (in parallel), then hipcc
links the shared library next to this file.  Always rebuilds.

``build(out=..., defines=[...], build_dir=...)`` makes a variant build with
extra ``-D`` macros (the kernels' tile parameters) at another path.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpagedattn.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["cache.hip", "decode.hip", "prefill.hip", "noalloc.hip"]
CXX_SOURCES = ["abi.cpp", "pool.cpp", "plan.cpp", "prefix.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 instructions are disabled for every device compile.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Fast math for the attention kernels.  The cache writes stay IEEE: the int8
# codes are decided by a float64 division and rounding that must be exact.
FAST_MATH = ["-ffast-math", "-fno-finite-math-only"]
PRECISE_SOURCES = {"cache.hip"}


def _hipcc():
    path = os.path.join(ROCM, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _compile(src, build_dir, extra):
    path = os.path.join(CSRC, src)
    obj = os.path.join(build_dir, src + ".o")
    if src.endswith(".hip"):
        fp = [] if src in PRECISE_SOURCES else FAST_MATH
        cmd = [_hipcc(), "-c", *COMMON, *HIP_FLAGS, *fp, *extra, path, "-o", obj]
    else:
        cmd = [_hipcc(), "-c", "-x", "c++", *COMMON, *extra, f"-I{ROCM}/include",
               "-D__HIP_PLATFORM_AMD__", path, "-o", obj]
    return src, cmd, subprocess.run(cmd, capture_output=True, text=True), obj


def build(verbose=False, out=None, defines=(), build_dir=None):
    lib = out or LIB
    build_dir = build_dir or BUILD
    os.makedirs(build_dir, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        results = list(pool.map(lambda s: _compile(s, build_dir, extra), HIP_SOURCES + CXX_SOURCES))
    objs = []
    for src, cmd, res, obj in results:
        noise = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
        if res.returncode != 0:
            raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{noise}")
        if verbose and noise.strip():
            print(noise, file=sys.stderr)
        objs.append(obj)
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
