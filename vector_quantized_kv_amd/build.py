"""Builds libvq.so (all HIP sources, gfx950) into the package directory.

Each source is compiled in two passes, in parallel across sources:
  1. device pass (--cuda-device-only): the gfx950 code object, bundled, with
     the device-only code-generation flags;
  2. host pass (--cuda-host-only): the host stubs, embedding that bundle.
The host objects are then linked into one shared library.  Splitting the
passes keeps the device-only target feature off the x86 host pass (where it
is not a known feature), and lets the sources compile concurrently.

Usage: python -m vector_quantized_kv_amd.build   (or build_library() from Python)
"""
from __future__ import annotations

import glob
import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libvq.so")
OBJDIR = os.path.join(os.path.dirname(PKG), "_build")
ARCH = "gfx950"

COMMON_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
                "-Wall", "-Wno-unused-function"]
DEVICE_FLAGS = [
    # never emit packed fp32 VALU ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # results of the matrix instructions in ordinary VGPRs (no accvgpr reads)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def clang() -> str:
    for cand in (os.environ.get("HIP_CLANG"), "/opt/rocm/lib/llvm/bin/clang++",
                 shutil.which("amdclang++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("ROCm clang++ not found (ROCm is required to build libvq)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.stdout or r.stderr:
        print(r.stdout + r.stderr, end="", flush=True)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)


def _compile(src, cc, verbose):
    name = os.path.splitext(os.path.basename(src))[0]
    # one compilation-unit id for both passes, so that the host's shadows of
    # file-scope device variables name the device pass's symbols
    cuid = hashlib.sha1(name.encode()).hexdigest()[:16]
    fatbin = os.path.join(OBJDIR, name + ".hipfb")
    obj = os.path.join(OBJDIR, name + ".o")
    _run([cc, *COMMON_FLAGS, *DEVICE_FLAGS, f"-cuid={cuid}", "--cuda-device-only", "-c", src,
          "-o", fatbin], verbose)
    _run([cc, *COMMON_FLAGS, f"-cuid={cuid}", "--cuda-host-only", "-c", src, "-o", obj,
          "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin], verbose)
    return obj


def build_library(verbose: bool = True) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    os.makedirs(OBJDIR, exist_ok=True)
    cc = clang()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, cc, verbose), srcs))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "--driver-mode=g++", "--hip-link", "-shared", "-fPIC",
          *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build_library()
    sys.exit(0)
