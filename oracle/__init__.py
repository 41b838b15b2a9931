"""CPU oracle for the BF16 x FP4 (NVFP4 / MXFP4) block-scaled GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``mixed_precision_bf16_amd``) never imports, calls or links anything here, and
nothing here imports the product path: the two share no code.

Everything is plain NumPy in float64, written from the definitions on the
pages (see the docstrings of ``oracle.fp4_oracle`` for the passage each
function follows).
"""

from .fp4_oracle import (  # noqa: F401
    E2M1_MAGNITUDES,
    FMT_MXFP4,
    FMT_NVFP4,
    bf16_bits_to_f64,
    bf16_bits_of_exact,
    check_tolerance,
    dequant_weights,
    e2m1_value,
    e4m3_value,
    e8m0_value,
    fp16_bits_of_exact,
    fp16_bits_to_f64,
    act_bits_to_f64,
    gemm_reference,
    group_size,
    scale_value,
    unpack_codes,
)
from .moe_oracle import moe_reference  # noqa: F401,E402
from .quant_oracle import native_reference, quantize_reference, scaled_gemm_reference  # noqa: F401,E402
