"""Build the HIP library (libvrc.so) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvrc.so")
# One translation unit per element type holds that type's kernels; vrc_api.hip
# holds the C ABI.  They compile in parallel.
SOURCES = [os.path.join(CSRC, f) for f in
           ("vrc_type_bf16.hip", "vrc_type_f16.hip", "vrc_type_f32.hip", "vrc_type_i32.hip", "vrc_api.hip")]
OBJDIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # Adds only, but never let the compiler contract or reassociate them.
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    # Keep packed-fp32 instructions out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


C_CHECK_SRC = os.path.join(ROOT, "tests", "c", "vrc_c_check.c")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c", "vrc_c_check")


def build_c_check(verbose: bool = False) -> str:
    """Build the plain-C user of the ABI (tests/c/vrc_c_check.c) against
    libvrc.so and /opt/rocm's HIP runtime."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", INCLUDE,
           "-o", C_CHECK_BIN, C_CHECK_SRC, "-L", PKG, "-lvrc", "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../ring_all_reduce_virtual_amd", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return C_CHECK_BIN


CVT_CHECK_SRC = os.path.join(ROOT, "tests", "c", "bf16_cvt_check.hip")
CVT_CHECK_BIN = os.path.join(ROOT, "tests", "c", "bf16_cvt_check")


def build_cvt_check(verbose: bool = False) -> str:
    """Build the exhaustive check of the bf16 conversion the kernels use
    (tests/c/bf16_cvt_check.hip), with the library's compiler flags."""
    flags = [f for f in FLAGS if f not in ("-fPIC", "-fvisibility=hidden")]
    cmd = [HIPCC, *flags, "-o", CVT_CHECK_BIN, CVT_CHECK_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return CVT_CHECK_BIN


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source to an object (in parallel) and link libvrc.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    objs, pending = [], []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        pending.append(cmd)
    running = []
    failed = None
    while pending or running:
        while pending and len(running) < jobs:
            cmd = pending.pop(0)
            running.append((cmd, subprocess.Popen(cmd)))
        cmd, proc = running.pop(0)
        if proc.wait() != 0 and failed is None:
            failed = cmd
    if failed is not None:
        raise subprocess.CalledProcessError(1, failed)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    build_c_check(verbose=True)
    build_cvt_check(verbose=True)
    sys.exit(0)
