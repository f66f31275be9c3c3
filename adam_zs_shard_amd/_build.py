"""Compile libzshard.so in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "build")
LIB_PATH = os.path.join(HERE, "libzshard.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# No FMA contraction anywhere, packed-fp32 instructions off, IEEE division
# and square root (the HIP defaults, stated), denormals kept (the default).
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-I", os.path.join(ROOT, "include"),
]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = ["zs_kernels.hip", "zs_capi.cpp"]
# Host-only code (the CPU offload update), compiled as plain C++: SIMD code
# paths are selected per function with target attributes.
HOST_SOURCES = ["zs_cpu.cpp"]
CXX = os.environ.get("CXX_HOST", "g++")
HOST = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off", "-fno-fast-math",
        "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        cmd = [CXX, *HOST, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build()
