"""Build libmlaverify.so in-tree (gfx950 device code + host C-ABI).

Usage: python -m mla_absorbed_tree_amd.build_lib [--resource-usage]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmlaverify.so")
ARCH = "gfx950"

HIP_SOURCES = ["verify_attn.hip", "kv_compact.hip", "tree_accept.hip"]
CXX_SOURCES = ["plan.cpp", "capi.cpp"]

# Packed fp32 VALU forms are kept out of the generated code on purpose.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-Wall", "-Wno-unused-variable"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libmlaverify needs ROCm to build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError("build step failed:\n%s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out)
    return out


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile every source and link libmlaverify.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
        out = _run([hipcc, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj],
                   verbose or resource_usage)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, resource_usage="--resource-usage" in sys.argv)
