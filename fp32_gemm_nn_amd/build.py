"""Build the HIP library fp32_gemm_nn_amd/libmisgemm.so for gfx950.

hipcc cross-compiles the device code without a GPU present. Packed-FP32 VALU
instructions are switched off for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "misgemm.hip")
LIB = os.path.join(PKG, "libmisgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    cmd = [HIPCC, *FLAGS, *(extra or []), SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    extra = [a for a in sys.argv[1:] if a != "-v"]
    print(build(verbose="-v" in sys.argv, extra=extra))
