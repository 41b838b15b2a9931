"""Plain float64 oracle of Y = A . dequant(W)^T for block-scaled FP4 weights.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
uses this module.

What is computed, and where the pages say so
--------------------------------------------
* A is BF16 activations, W holds FP4 weight codes with block scales, Y is the
  BF16 product accumulated in higher precision ("Optimizing FP4
  Mixed-Precision Inference on AMD GPUs", the Petit blog, translated on
  winzheng.com / winzheng.jp: introduction and section "Efficient
  dequantization through preprocessing": FP16/BF16 x FP4 kernels that
  dequantize FP4 weights to BF16/FP16 and use the BF16 matrix cores).
* FP4 is E2M1: one sign, two exponent and one mantissa bit; the positive
  non-zero values are 0.5, 1, 1.5, 2, 3, 4, 6; with sign and zero 16 states
  (mhpq.cn FP4 GEMM article, section 2.1).
* Block scaling: each block of consecutive elements shares one scale and the
  stored codes are the data divided by that scale (same article, section 2.2),
  so the weight value is code value x scale.
* NVFP4: 16 elements share one FP8 scale (Petit blog, section "Detailed
  performance analysis"); read here as OCP FP8 E4M3 ("E4M3FN": bias 7, no
  infinities, S.1111.111 is NaN).
* MXFP4: named as a supported weight format (petit-kernel PyPI page,
  "Features"); read here as the OCP MX definition: 32 elements share one E8M0
  scale 2^(b - 127), byte 0xFF is NaN.
* Scales are positive and codes contain no negative zero (petit-kernel PyPI
  page, "Known limitations"); the oracle still decodes those values (a
  negative-zero code is -0.0, a negative scale is negative) so it can judge any
  input.

Storage conventions (read where the pages are silent)
-----------------------------------------------------
* A: uint16 array [m][K] of BF16 bit patterns, row-major (or FP16 bit
  patterns for the FP16-activation variant of the same kernels, which the
  Petit blog's introduction names alongside BF16).
* codes: uint8 array [N][K/2]; byte j of row n holds element k = 2j in bits
  3..0 and k = 2j + 1 in bits 7..4 (two FP4 values per byte, mhpq.cn article
  section 3.3; which nibble comes first is not stated).
* scales: uint8 array [N][K/G]; byte g of row n scales elements
  k in [g*G, (g+1)*G) (scales laid out along K, mhpq.cn article section 3.3).

Pins: see ``tests/test_oracle.py`` (E2M1 value list of the page, library FP8
decoders, exact rational brute force, hand-worked examples, closed-form
exactness of every code x scale product in BF16).
"""

from __future__ import annotations

import numpy as np

FMT_NVFP4 = 0
FMT_MXFP4 = 1

# Positive E2M1 magnitudes in code order 0..7 (mhpq.cn article, section 2.1
# lists exactly these non-zero values).  The decode below derives them from the
# sign/exponent/mantissa fields; this tuple is only used for documentation and
# is cross-checked by the tests.
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def group_size(fmt: int) -> int:
    """Elements per scale: 16 for NVFP4 (Petit blog, "Detailed performance
    analysis"), 32 for MXFP4 (OCP MX reading of the petit-kernel format)."""
    if fmt == FMT_NVFP4:
        return 16
    if fmt == FMT_MXFP4:
        return 32
    raise ValueError(f"unknown FP4 format {fmt}")


def e2m1_value(code):
    """Value of a 4-bit E2M1 code (mhpq.cn article, section 2.1).

    Fields: sign = bit 3, exponent = bits 2..1, mantissa = bit 0.  With
    exponent bias 1 and exponent 0 read as subnormal, the positive codes decode
    to 0, 0.5, 1, 1.5, 2, 3, 4, 6, the value list the page gives; no other bias
    produces that list, which fixes the reading.
    """
    c = np.asarray(code, dtype=np.int64)
    sign = (c >> 3) & 1
    exp = (c >> 1) & 3
    man = c & 1
    subnormal = man * 0.5                                   # 0.m x 2^(1-1)
    normal = (1.0 + man / 2.0) * np.exp2(exp.astype(np.float64) - 1.0)
    mag = np.where(exp == 0, subnormal, normal)
    return np.where(sign == 1, -mag, mag).astype(np.float64)


def e4m3_value(byte):
    """OCP FP8 E4M3 (E4M3FN) decode: the NVFP4 "FP8 scale" of the Petit blog,
    section "Detailed performance analysis".

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0;
    exponent 0 is subnormal (f/8 x 2^-6); S.1111.111 is NaN; no infinities.
    """
    b = np.asarray(byte, dtype=np.int64)
    sign = (b >> 7) & 1
    exp = (b >> 3) & 15
    man = b & 7
    subnormal = (man / 8.0) * 2.0 ** -6
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag).astype(np.float64)


def e8m0_value(byte):
    """OCP MX E8M0 scale decode: 2^(b - 127); 0xFF is NaN."""
    b = np.asarray(byte, dtype=np.int64)
    val = np.exp2(b.astype(np.float64) - 127.0)
    return np.where(b == 255, np.nan, val)


def scale_value(byte, fmt: int):
    """Decode scale bytes of either format."""
    if fmt == FMT_NVFP4:
        return e4m3_value(byte)
    if fmt == FMT_MXFP4:
        return e8m0_value(byte)
    raise ValueError(f"unknown FP4 format {fmt}")


def unpack_codes(codes: np.ndarray, K: int) -> np.ndarray:
    """[N][K/2] packed bytes -> [N][K] codes 0..15 (element 2j = low nibble)."""
    codes = np.asarray(codes, dtype=np.uint8)
    N = codes.shape[0]
    if codes.shape[1] * 2 != K:
        raise ValueError("codes must have K/2 bytes per row")
    out = np.empty((N, K), dtype=np.int64)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def dequant_weights(codes: np.ndarray, scales: np.ndarray, K: int, fmt: int) -> np.ndarray:
    """W[n][k] = E2M1(code[n][k]) x scale[n][k // G] in float64.

    This is the block-scaling definition of the mhpq.cn article, section 2.2,
    read backwards (stored code x block scale).  The product is exact in
    float64 and, for the scales the pages allow, exact in BF16 too.
    """
    G = group_size(fmt)
    if K % G != 0:
        raise ValueError(f"K={K} must be a multiple of the group size {G}")
    scales = np.asarray(scales, dtype=np.uint8)
    if scales.shape != (np.asarray(codes).shape[0], K // G):
        raise ValueError("scales must have K/G bytes per row")
    vals = e2m1_value(unpack_codes(codes, K))
    s = scale_value(scales, fmt)                      # [N][K/G]
    return vals * np.repeat(s, G, axis=1)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float64 (exact: BF16 is the top half of FP32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_bits_of_exact(values: np.ndarray) -> np.ndarray:
    """BF16 bit patterns of float64 values that are exactly representable in
    BF16; raises if any value is not (used for the bit-exact dequant check)."""
    v = np.asarray(values, dtype=np.float64)
    f = v.astype(np.float32)
    bits = f.view(np.uint32)
    finite = np.isfinite(v)
    bad = finite & ((f.astype(np.float64) != v) | ((bits & 0xFFFF) != 0))
    if np.any(bad):
        raise ValueError("value not exactly representable in BF16")
    return (bits >> 16).astype(np.uint16)


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64, decoded from the fields:
    sign = bit 15, exponent = bits 14..10 (bias 15), mantissa = bits 9..0;
    exponent 0 is subnormal (f/1024 x 2^-14), exponent 31 is Inf (f = 0) or
    NaN."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = (b >> 15) & 1
    exp = (b >> 10) & 31
    man = b & 1023
    subnormal = (man / 1024.0) * 2.0 ** -14
    normal = (1.0 + man / 1024.0) * np.exp2(exp.astype(np.float64) - 15.0)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where(exp == 31, np.where(man == 0, np.inf, np.nan), mag)
    return np.where(sign == 1, -mag, mag).astype(np.float64)


def fp16_bits_of_exact(values: np.ndarray) -> np.ndarray:
    """FP16 bit patterns of float64 values that are exactly representable in
    FP16; raises if any value is not."""
    v = np.asarray(values, dtype=np.float64)
    h = v.astype(np.float16)
    finite = np.isfinite(v)
    if np.any(finite & (h.astype(np.float64) != v)):
        raise ValueError("value not exactly representable in FP16")
    return h.view(np.uint16)


def act_bits_to_f64(bits: np.ndarray, act: str = "bf16") -> np.ndarray:
    """Activation / output bit patterns (BF16 or FP16) -> float64."""
    if act == "bf16":
        return bf16_bits_to_f64(bits)
    if act == "f16":
        return fp16_bits_to_f64(bits)
    raise ValueError(f"unknown activation type {act}")


GEMM_CHUNK_ROWS = 2048


def gemm_reference(a_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                   K: int, fmt: int, act: str = "bf16"):
    """Y_ref[i][n] = sum_k a[i][k] w[n][k] and B[i][n] = sum_k |a[i][k] w[n][k]|.

    Both in float64 with a library matrix product (the error of the float64 sum
    is below K * 2^-53 * B, negligible against the tolerance).  `act` names
    the type of the activation bits (BF16 or FP16).  Returns (y_ref, bound),
    each [m][N].

    The weight rows are dequantized and multiplied GEMM_CHUNK_ROWS at a time
    (a plain loop over N that only bounds memory: every output column is the
    same dot product over all of K whatever the chunking).
    """
    a = act_bits_to_f64(a_bits, act)
    if a.ndim != 2 or a.shape[1] != K:
        raise ValueError("A must be [m][K]")
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    N = codes.shape[0]
    y = np.empty((a.shape[0], N), dtype=np.float64)
    bound = np.empty((a.shape[0], N), dtype=np.float64)
    abs_a = np.abs(a)
    for n0 in range(0, N, GEMM_CHUNK_ROWS):
        n1 = min(N, n0 + GEMM_CHUNK_ROWS)
        w = dequant_weights(codes[n0:n1], scales[n0:n1], K, fmt)
        y[:, n0:n1] = a @ w.T
        bound[:, n0:n1] = abs_a @ np.abs(w).T
    return y, bound


def check_tolerance(y_bits: np.ndarray, y_ref: np.ndarray, bound: np.ndarray,
                    rel: float = 8e-3, abs_of_bound: float = 2e-3, act: str = "bf16") -> np.ndarray:
    """Element-wise pass mask: y finite and |y - y_ref| <= rel*|y_ref| + abs_of_bound*B.

    The bound covers BF16 round-to-nearest of the output (<= 2^-9 relative;
    FP16: 2^-11) plus any FP32 summation order over K <= 33554 terms
    (<= K 2^-24 B).
    """
    y = act_bits_to_f64(y_bits, act)
    err = np.abs(y - y_ref)
    return np.isfinite(y) & (err <= rel * np.abs(y_ref) + abs_of_bound * bound)
