"""Build the HIP library ``libslot_kv.so`` in-tree for gfx950.

    python -m sequence_slot_kv_amd.build          # compile
    python -m sequence_slot_kv_amd.build --check  # print per-kernel register use

The library is compiled with hipcc directly (no torch extension machinery):
the C ABI in include/slot_kv.h is the product, and the Python binding loads it
with ctypes.  Packed FP32 instructions are disabled for every kernel.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libslot_kv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["slot_kv_api.hip", "slot_kv_kernels.hip", "slot_kv_prefill.hip", "slot_kv_state.hip",
           "slot_kv_plan.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # every atomic in the kernels is issued by a single lane; the
          # wave-aggregating rewrite would read each result at once
          "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
          "-I", INCLUDE, "-I", CSRC]


def build(extra=None, out: str = LIB, verbose: bool = False) -> str:
    """Compile every source into ``out`` (a fresh build each call)."""
    extra = list(extra or [])
    tmp = out + ".tmp"
    cmd = [HIPCC, *COMMON, *extra, "-shared", "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def resource_usage() -> str:
    """Per-kernel VGPR / SGPR / LDS / occupancy report from the compiler."""
    cmd = [HIPCC, *COMMON, "--cuda-device-only", "-c", "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage",
           os.path.join(CSRC, "slot_kv_kernels.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr)
    return r.stderr


if __name__ == "__main__":
    if "--check" in sys.argv:
        print(resource_usage())
    else:
        print(build(verbose=True))
