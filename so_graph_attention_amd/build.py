"""Build libe2a.so (HIP, gfx950) and the host-only geometry check library in-tree.

Usage:  python -m so_graph_attention_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
OBJDIR = os.path.join(PKG, "_build")
ROOT = os.path.dirname(PKG)

ARCH = os.environ.get("E2A_OFFLOAD_ARCH", "gfx950")
HIP_SOURCES = ["e2a_api.hip", "neighbors.hip", "attention_reference.hip", "attention_mfma.hip",
               "attention_backward.hip", "attention_wgrad.hip", "block.hip"]
# Packed fp32 VALU forms are kept off for every HIP translation unit.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]
PER_FILE = {"neighbors.hip": ["-ffp-contract=off"]}


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(OBJDIR, exist_ok=True)
    hipcc = _hipcc()

    def compile_one(src):
        obj = os.path.join(OBJDIR, src + ".o")
        _run([hipcc, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(HIP_SOURCES))) as ex:
        objs = list(ex.map(compile_one, HIP_SOURCES))
    lib = os.path.join(LIBDIR, "libe2a.so")
    tmp = lib + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, lib)
    # host-only build of the per-edge geometry routines (CPU checks of the recursion)
    hlib = os.path.join(LIBDIR, "libe2a_hostgeom.so")
    _run(["g++", "-O2", "-shared", "-fPIC", "-std=c++17", os.path.join(CSRC, "host_geometry.cpp"),
          "-o", hlib + ".tmp"])
    os.replace(hlib + ".tmp", hlib)
    if verbose:
        print("built", lib, "and", hlib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
