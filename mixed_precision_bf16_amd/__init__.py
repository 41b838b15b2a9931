"""BF16 x FP4 (NVFP4 / MXFP4) block-scaled GEMM for AMD MI355X (gfx950).

The computation lives in a C-ABI shared library (``libfp4gemm.so``, built
from ``csrc/`` by ``build.py``); ``fp4gemm`` is the thin ctypes binding over
it.  ``synth`` draws seeded synthetic inputs.
"""
