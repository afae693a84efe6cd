"""Build libtreeattn.so in-tree for gfx950 with hipcc.

Usage: ``python -m shared_prefix_tree_parent_amd.build_lib`` (or ``build()`` from Python).
Every call recompiles.  Objects go to ``_build/`` at the repository root; the library is
written next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtreeattn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for all device code (the compiler would otherwise form
# them from ordinary float code).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]

HIP_SOURCES = ["classify.hip", "attn_fwd.hip", "attn_bwd.hip", "rope.hip", "gdn.hip", "capi.hip"]
# Per-source device flags.  The backward and the GDN scan keep every MFMA result in ordinary
# VGPRs: their softmax or decay work reads the score MFMAs' results, and with the default
# accumulator-register form each result is copied back to a VGPR first (one extra VALU op per
# value).
SOURCE_FLAGS = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "gdn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
CXX_SOURCES = ["plan.cpp"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + p.stdout)
    return p.stdout


def build(verbose: bool = False, save_temps: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd.insert(1, "-save-temps=obj")
        jobs.append((cmd, obj))
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cxx = shutil.which("g++") or "g++"
        jobs.append(([cxx, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    if verbose:
        for (cmd, _), out in zip(jobs, outs):
            print(" ".join(cmd))
            if out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for _, o in jobs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv))
