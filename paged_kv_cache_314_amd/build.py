"""Build libpagedattn.so (HIP kernels for gfx950 + host planner + C ABI) in-tree.

    python -m paged_kv_cache_314_amd.build        # or build() from Python

hipcc compiles the .hip sources for gfx950 only; the host planner (plan.cpp) is
plain C++17 built with g++, so it is visibly free of HIP calls.  Objects go to
paged_kv_cache_314_amd/_build/, the library to paged_kv_cache_314_amd/.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedattn.so")

HIP_SOURCES = ["api.hip", "decode.hip", "prefill.hip", "fill.hip", "append.hip"]
CXX_SOURCES = ["plan.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms are not used (compiler would otherwise emit them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def _compile(src):
    base = os.path.splitext(src)[0]
    obj = os.path.join(BUILD, base + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC] + HIP_FLAGS + ["-c", path, "-o", obj]
    else:
        cmd = ["g++"] + CXX_FLAGS + ["-c", path, "-o", obj]
    _run(cmd)
    return obj


def build(verbose=False):
    """Compile every source and link the shared library.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    sources = HIP_SOURCES + CXX_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
