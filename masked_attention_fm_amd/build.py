"""Build libflashmask.so (all HIP sources, gfx950 only) in-tree.

    python -m masked_attention_fm_amd.build [--verbose]

hipcc cross-compiles without a GPU.  The library lands at
masked_attention_fm_amd/lib/libflashmask.so, next to the binding that loads it.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libflashmask.so")

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    # No packed fp32 arithmetic: the compiler must not form v_pk_{add,mul,fma}_f32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libflashmask")
    return path


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs = []
    procs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *HIP_FLAGS, "-c", src, "-o", obj]
        if resource_usage:
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        # The host pass does not know the packed-fp32 feature; that note is harmless.
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or resource_usage or p.returncode != 0):
            print("\n".join(lines), flush=True)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed on: " + ", ".join(failed))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv, resource_usage="--resources" in sys.argv)
    print(LIB)
