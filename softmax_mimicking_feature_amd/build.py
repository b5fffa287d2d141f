"""Build libhh.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m softmax_mimicking_feature_amd.build

Every source under csrc/ is compiled in parallel and linked into
softmax_mimicking_feature_amd/libhh.so.  All device code is built with packed
fp32 instructions disabled (-packed-fp32-ops).
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
LIB = os.path.join(PKG, "libhh.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("HH_OFFLOAD_ARCH", "gfx950")

SOURCES = ["hh_api.cpp", "hh_wide.hip", "hh_narrow.hip", "hh_misc.hip", "hh_distill.hip", "hh_noalloc.hip", "hh_feat.hip", "hh_bwd.hip"]


def _hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libhh")


def _flags(src: str):
    f = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Wall", "-Wno-unused-function", "-Wno-unused-result"]
    if src.endswith(".hip"):
        f += ["-x", "hip", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-ffp-contract=fast", "-munsafe-fp-atomics"]
    return f


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + _flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = [ln for ln in (r.stdout + r.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n" + "\n".join(noise))
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
