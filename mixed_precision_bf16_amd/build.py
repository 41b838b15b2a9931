"""Build ``libfp4gemm.so`` in-tree with hipcc for gfx950.

    python -m mixed_precision_bf16_amd.build

The library is compiled every time this runs (seconds).  Tests, ``bench.py``
and the smoke entry load the built file and only build when it is absent.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libfp4gemm.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["repack.cpp", "fp4gemm.hip"]
HEADERS = ["layout.h", os.path.join("..", "..", "include", "fp4gemm.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 instructions are kept out of every kernel (compiler feature off).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950", "-Wall",
          "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    """Compile the shared library; returns its path.  Raises on failure."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def ensure_built() -> str:
    """Path of the library, building it only when it does not exist yet."""
    if not os.path.exists(LIB_PATH):
        build()
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
