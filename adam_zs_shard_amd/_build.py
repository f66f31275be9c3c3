"""Compile libzshard.so in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "build")
LIB_PATH = os.path.join(HERE, "libzshard.so")
# bandwidth probes for bench.py --ceiling: a separate library, not the step
PROBE_PATH = os.path.join(HERE, "libzsprobe.so")
PROBE_SOURCES = ["zs_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# No FMA contraction anywhere, packed-fp32 instructions off, IEEE division
# and square root (the HIP defaults, stated), denormals kept (the default).
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-I", os.path.join(ROOT, "include"),
]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# Device code is split over several translation units (the fused kernels per
# gradient dtype) so that they compile in parallel.
SOURCES = ["zs_fused_f16.hip", "zs_fused_bf16.hip", "zs_table.hip", "zs_unfused.hip",
           "zs_common.hip", "zs_capi.cpp", "zs_offload.cpp"]
# Host-only code (the CPU offload update), compiled as plain C++: SIMD code
# paths are selected per function with target attributes.
HOST_SOURCES = ["zs_cpu.cpp"]
CXX = os.environ.get("CXX_HOST", "g++")
HOST = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off", "-fno-fast-math",
        "-I", os.path.join(ROOT, "include")]


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(8, n))


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        cmds.append([HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src),
                     "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        cmds.append([CXX, *HOST, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    probe_objs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        cmds.append([HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src),
                     "-o", obj])
        probe_objs.append(obj)
    # every translation unit at once, at most _jobs() compilers running
    running, failed = [], []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        running.append((cmd, subprocess.Popen(cmd)))
        while sum(p.poll() is None for _, p in running) >= _jobs():
            running[[p.poll() is None for _, p in running].index(True)][1].wait()
    for cmd, p in running:
        if p.wait() != 0:
            failed.append(cmd[-3])  # the source file
    if failed:
        raise subprocess.CalledProcessError(1, failed)
    for path, ob in ((LIB_PATH, objs), (PROBE_PATH, probe_objs)):
        tmp = path + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *ob]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    build()
