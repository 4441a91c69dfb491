"""Build libpagedattn.so in-tree for gfx950.

Run ``python -m paged_kv_cache_block_amd.build`` (or ``__graft_entry__.build()``).
Each source compiles to an object in ``_build/`` (in parallel), then hipcc
links the shared library next to this file.  Always rebuilds.
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

HIP_SOURCES = ["cache.hip", "decode.hip", "prefill.hip"]
CXX_SOURCES = ["abi.cpp", "pool.cpp", "plan.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 instructions are disabled for every device compile.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffast-math", "-fno-finite-math-only"]


def _hipcc():
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src):
    hipcc = _hipcc()
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc, "-c", *COMMON, *HIP_FLAGS, path, "-o", obj]
    else:
        rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
        cmd = [hipcc, "-c", "-x", "c++", *COMMON, f"-I{rocm}/include", "-D__HIP_PLATFORM_AMD__",
               path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    return src, cmd, res, obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        for src, cmd, res, obj in pool.map(_compile, HIP_SOURCES + CXX_SOURCES):
            noise = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                              if "packed-fp32-ops" not in l)
            if res.returncode != 0:
                raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{noise}")
            if verbose and noise.strip():
                print(noise, file=sys.stderr)
            objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
