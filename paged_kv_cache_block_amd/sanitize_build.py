"""A host-sanitized build of libpagedattn.so, for testing on a CPU machine.

The host bookkeeping translation units (pool, plan, prefix cache and the C
ABI layer) are compiled with AddressSanitizer and UndefinedBehaviorSanitizer
by ROCm's clang++ (host code only; every undefined behaviour is fatal), the
HIP sources as in the normal build, and the library is linked against
clang's shared sanitizer runtime.  A process that loads it must preload that
runtime (``runtime_library()``), e.g.::

    LD_PRELOAD=$(runtime) ASAN_OPTIONS=detect_leaks=0 python ...

``build_sanitized()`` returns the path of the library (under
``_build/sanitize/``, never next to the normal one).
"""

from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from . import build as _build

OUT_DIR = os.path.join(_build.ROOT, "_build", "sanitize")
LIB = os.path.join(OUT_DIR, "libpagedattn_sanitized.so")

# Host-only compile and link flags of the sanitized translation units.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _clangxx():
    path = os.path.join(_build.ROCM, "llvm", "bin", "clang++")
    return path if os.path.exists(path) else "clang++"


def runtime_library():
    """Path of clang's shared AddressSanitizer runtime (with the UBSan handlers)."""
    pattern = os.path.join(_build.ROCM, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")
    found = sorted(glob.glob(pattern))
    if not found:
        raise FileNotFoundError(f"no clang AddressSanitizer runtime matches {pattern}")
    return found[-1]


def _host_compile(src):
    path = os.path.join(_build.CSRC, src)
    obj = os.path.join(OUT_DIR, src + ".o")
    cmd = [_clangxx(), "-c", "-x", "c++", "-O1", "-g", "-std=c++17", "-fPIC", "-Wall", *SANITIZE,
           f"-I{_build.INCLUDE}", f"-I{_build.CSRC}", f"-I{_build.ROCM}/include", "-D__HIP_PLATFORM_AMD__",
           path, "-o", obj]
    return src, cmd, subprocess.run(cmd, capture_output=True, text=True), obj


def build_sanitized():
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        hip = list(pool.map(lambda s: _build._compile(s, OUT_DIR, []), _build.HIP_SOURCES))
        host = list(pool.map(_host_compile, _build.CXX_SOURCES))
    objs = []
    for src, cmd, res, obj in hip + host:
        if res.returncode != 0:
            raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [_clangxx(), "-shared", "-fPIC", *SANITIZE, "-shared-libsan", *objs,
           f"-L{_build.ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{_build.ROCM}/lib",
           f"-Wl,-rpath,{os.path.dirname(runtime_library())}", "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_sanitized())
