"""Compile the HIP library in-tree for gfx950 (hipcc, no JIT cache).

Produces ``sliding_window_cached_amd/libvrt.so`` from ``csrc/``.  The whole
library is built with ``-ffp-contract=off`` (every fused multiply-add in the
kernels is written out, so two builds or two template instantiations round
identically) and without packed-fp32 instructions.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libvrt.so")
ARCH = os.environ.get("VRT_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
DEVICE = [
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the softmax works on the
    # score tiles in place instead of copying them out of AGPRs every tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src, is_hip in (("vrt_host.cpp", False), ("vrt_kernels.hip", True), ("vrt_mfma.hip", True),
                        ("vrt_block.hip", True), ("vrt_probe.hip", True)):
        obj = os.path.join(out_dir, src + ".o")
        cmd = [hipcc, "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
        cmd += (["-x", "hip"] + DEVICE) if is_hip else ["-D__HIP_PLATFORM_AMD__"]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
