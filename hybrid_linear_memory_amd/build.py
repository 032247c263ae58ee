"""Build libarl2.so in-tree with hipcc for gfx950.

    python -m hybrid_linear_memory_amd.build      # or __graft_entry__.build()

The library is one shared object: the C-ABI layer (csrc/api.cpp) plus the
HIP kernels (csrc/*.hip), compiled for gfx950 only. All HIP code is built
without packed-fp32 instruction selection.
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
LIB = os.path.join(PKG, "libarl2.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "kernels_generic.hip", "kernels_mfma.hip", "kernels_token.hip",
           "kernels_train.hip", "noalloc.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libarl2")
    return path


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object (in parallel) and link libarl2.so."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if out.returncode != 0:
        raise RuntimeError(f"link of libarl2.so failed:\n{out.stdout}")
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out.decode(errors='replace')}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
