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
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libslot_kv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["slot_kv_api.hip", "slot_kv_kernels.hip", "slot_kv_prefill.hip", "slot_kv_state.hip",
           "slot_kv_plan.cpp"]

def common(csrc: str = CSRC) -> list:
    """hipcc flags of every source (headers from ``csrc``)."""
    return ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # every atomic in the kernels is issued by a single lane; the
            # wave-aggregating rewrite would read each result at once
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-I", INCLUDE, "-I", csrc]


COMMON = common()

# Flags of single sources.  The prefill kernels keep their MFMA accumulators
# in ordinary VGPRs: in the AGPR form every rescale of an output accumulator
# copies it out and back, and the split register file lowers the tiled
# attention's occupancy from four waves per SIMD to three.
PER_SOURCE = {"slot_kv_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(extra=None, out: str = LIB, verbose: bool = False, csrc: str = CSRC) -> str:
    """Compile every source of ``csrc`` (in parallel) and link ``out``; a
    fresh build each call."""
    extra = list(extra or [])
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory() as tmpd:
        jobs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpd, src + ".o")
            cmd = [HIPCC, *common(csrc), *PER_SOURCE.get(src, []), *extra, "-c", "-o", obj,
                   os.path.join(csrc, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            jobs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                               stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        failed = []
        for cmd, proc in jobs:
            so, se = proc.communicate()
            if proc.returncode != 0:
                failed.append(f"{cmd[-1]} ({proc.returncode}):\n{so}\n{se}")
        if failed:
            raise RuntimeError("hipcc failed: " + "\n".join(failed))
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
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
