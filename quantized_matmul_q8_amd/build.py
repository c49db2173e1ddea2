"""Build libqmm.so (the HIP kernels and the C ABI) in-tree for gfx950.

Runs hipcc once over every source in ``csrc/``.  Flags: ``-O3``, no fast
math (the Q8_1 quantizer must match IEEE fp32 bit for bit), packed fp32 VALU
instructions disabled for the device code, and MFMA results kept in VGPRs.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqmm.so")
ARCH = os.environ.get("QMM_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = LIB + ".tmp"
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results in VGPRs: the AGPR form made the epilogue copy every
        # int8-MFMA result back with accvgpr reads (one VALU op per element)
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}", "-o", tmp, *srcs,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libqmm.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
