"""Build libkvmove.so in-tree for gfx950 with hipcc.

The library is one shared object built from csrc/kernels.hip (device code)
and csrc/api.cpp (the extern "C" boundary), against include/kvm.h.
Packed-FP32 instruction selection is switched off for all HIP code.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvmove.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libkvmove")


def command(out: str = LIB, extra=()) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, *extra, "-o", out,
            os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "api.cpp")]


def build(out: str = LIB, extra=(), quiet: bool = True) -> str:
    tmp = out + ".tmp"
    res = subprocess.run(command(tmp, extra), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    if not quiet and res.stderr:
        print(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
