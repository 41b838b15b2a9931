"""Build ``libfp4gemm.so`` in-tree with hipcc for gfx950.

    python -m mixed_precision_bf16_amd.build

The library is compiled every time this runs (its translation units in
parallel, about a minute).  Tests, ``bench.py``
and the smoke entry load the built file and only build when it is absent.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libfp4gemm.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["repack.cpp", "fp4gemm.hip", "decode_bf16.hip", "decode_f16.hip", "prefill_bf16.hip", "prefill_f16.hip",
           "moe_bf16.hip"]
HEADERS = ["layout.h", "kernels.h", "dispatch.h", "decode_inst.inc", "prefill_inst.inc",
           os.path.join("..", "..", "include", "fp4gemm.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 instructions are kept out of every kernel (compiler feature off).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every translation unit (in parallel) and link the shared
    library; returns its path.  Raises on failure."""
    from concurrent.futures import ThreadPoolExecutor
    with tempfile.TemporaryDirectory(prefix="fp4gemm_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(src)[0] + ".o") for src in SOURCES]
        cmds = [[HIPCC, *COMMON, *DEVICE_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src),
                 "-o", obj] for src, obj in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB_PATH + ".tmp"
        _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def ensure_built() -> str:
    """Path of the library, building it only when it does not exist yet."""
    if not os.path.exists(LIB_PATH):
        build()
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
