"""Builds libpsw.so (host C++ with g++, HIP kernels with hipcc for gfx950).

Usage: ``python -m paged_sliding_window_append_amd.build`` (always rebuilds).
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so it travels with the package.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpsw.so")

ARCH = "gfx950"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CXX = shutil.which("g++") or "g++"

HOST_SOURCES = ["capi.cpp", "page_manager.cpp"]
HIP_SOURCES = ["kernels.hip", "attention.hip", "dense.hip", "scratch.hip"]

# Packed fp32 VALU instructions are kept out of every device build.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
# The attention kernel produces no NaNs (masked scores are -inf and every
# row sees at least one finite score first), so its max operations need no
# signalling-NaN quieting: IEEE mode off there.
FILE_FLAGS = {"attention.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    noise = "is not a recognized feature for this target"
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if noise not in line and line.strip())
    if out and verbose:
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([CXX, *HOST_FLAGS, "-I", INCLUDE, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([HIPCC, *HIP_FLAGS, *FILE_FLAGS.get(src, []), "-I", INCLUDE, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs,
          "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
