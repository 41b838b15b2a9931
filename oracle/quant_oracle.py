"""Plain oracle of the offline FP4 quantizer (BF16 weights -> E2M1 codes and
block scales) and of the per-tensor output scale alpha.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
uses this module.

What is computed, and where the pages say so
--------------------------------------------
* Block scaling (mhpq.cn FP4 GEMM article, section 2.2): each block of G
  consecutive K elements gets one scale, the block is divided by it and the
  quotients are quantized; the scale follows the block's maximum absolute
  value ("max-scaling").
* Each quotient goes to the nearest E2M1 grid point (same article, section
  2.1: 16 states, the positive non-zero values 0.5 ... 6).
* An all-zero block must not get a zero scale (same article, section 5.2:
  protect the scale with a small floor).
* Scales positive, no negative-zero codes (petit-kernel page, "Known
  limitations": what the offline transformation accepts).

Readings (the pages leave these open):
* NVFP4 block scale = E4M3 round-to-nearest-even of amax / 6 / alpha
  (the block maximum lands on the largest grid value), saturated to 448 and
  floored at the smallest positive E4M3 (2^-9), so it is never zero.
* MXFP4 block scale = 2^(floor(log2(amax / alpha)) - 2) (the OCP MX rule for
  E2M1, whose largest exponent is 2), byte clamped to 0 .. 254.  Byte 0 is
  the scale 2^-127 like any other byte (it covers every amax / alpha below
  2^-124, including an all-zero block); its block is divided and rounded
  like every other block (section 2.2 of the article), so only elements
  that round to zero get code 0.
* An infinite amax gives the largest scale (E4M3 448, E8M0 byte 254).
* Effective scale S = alpha * scale; quotient q = |x| / S; nearest grid
  value with ties to the even mantissa bit (round-to-nearest-even), values
  beyond 6 saturate to 6; the sign bit is set only on non-zero codes.  NaN
  inputs give code 0 and infinities +-6.
* Arithmetic: every decision is taken in IEEE FP32 (amax / 6, / alpha,
  alpha * scale, |x| / S, each correctly rounded) so that the GPU quantizer
  and this oracle decide identically.
* alpha (the NVFP4 per-tensor second-level scale; not mentioned on the pages)
  multiplies the GEMM output: Y = alpha * A . dequant(W)^T.
"""

from __future__ import annotations

import numpy as np

from .fp4_oracle import bf16_bits_to_f64, e4m3_value, group_size

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_rne_byte(t: np.ndarray) -> np.ndarray:
    """Non-negative FP32 values -> E4M3 byte of the nearest representable
    value (ties to the even mantissa), saturating at 448 (byte 0x7E)."""
    return _nearest_in(np.asarray(t, dtype=np.float64), e4m3_value(np.arange(0, 0x7F))).astype(np.uint8)


def _nearest_in(x: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of the increasing table vals (ties to the
    even index; values past the last entry take the last index)."""
    hi = np.clip(np.searchsorted(vals, x, side="left"), 1, len(vals) - 1)
    lo = hi - 1
    dlo, dhi = np.abs(x - vals[lo]), np.abs(vals[hi] - x)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return np.where(x >= vals[-1], len(vals) - 1, pick)


def nearest_e2m1(q: np.ndarray) -> np.ndarray:
    """Non-negative quotients -> E2M1 magnitude code 0..7: nearest grid value,
    ties to the even code (even mantissa bit), saturating at 6; NaN -> 0."""
    q = np.asarray(q, dtype=np.float64)
    nan = np.isnan(q)
    return np.where(nan, 0, _nearest_in(np.where(nan, 0.0, q), GRID)).astype(np.int64)


def quantize_reference(w_bits: np.ndarray, fmt: int, alpha: float = 1.0):
    """BF16 weights [N][K] (bit patterns) -> (codes u8 [N][K/2], scales u8
    [N][K/G]) by the rules in the module docstring."""
    G = group_size(fmt)
    w = bf16_bits_to_f64(w_bits).astype(np.float32)            # exact
    N, K = w.shape
    if K % G:
        raise ValueError("K must be a multiple of the group size")
    a32 = np.float32(alpha)
    blocks = w.reshape(N, K // G, G)
    with np.errstate(invalid="ignore"):
        amax = np.nanmax(np.abs(blocks), axis=2, initial=np.float32(0)).astype(np.float32)
    if fmt == 0:
        t = (amax / np.float32(6.0)).astype(np.float32) / a32
        sb = e4m3_rne_byte(t.astype(np.float32))
        sb = np.where(sb == 0, 1, sb).astype(np.uint8)
        sval = e4m3_value(sb).astype(np.float32)
    else:
        t = (amax / a32).astype(np.float32)
        mant, ex = np.frexp(t.astype(np.float64))                # t = mant * 2^ex, mant in [0.5, 1)
        e = np.where(t > 0, ex - 1 - 2, -127)
        e = np.where(np.isinf(t), 127, e)
        sb = np.clip(e + 127, 0, 254).astype(np.uint8)
        sval = np.exp2(sb.astype(np.float64) - 127.0).astype(np.float32)   # byte 0: 2^-127, an FP32 subnormal
    S = (a32 * sval).astype(np.float32)                         # [N][K/G]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (np.abs(blocks) / S[..., None]).astype(np.float32)
    mag = nearest_e2m1(q)
    neg = np.signbit(blocks) & (mag != 0) & ~np.isnan(blocks)
    code = (mag | np.where(neg, 8, 0)).reshape(N, K).astype(np.uint8)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sb


def scaled_gemm_reference(y_ref: np.ndarray, bound: np.ndarray, alpha: float):
    """Y = alpha * (A . dequant(W)^T); the bound scales the same way."""
    a = float(np.float32(alpha))
    return a * y_ref, abs(a) * bound


def native_reference(a_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, K: int):
    """The native FP4 path (FP4 x FP4 on the matrix cores; the Petit blog's
    introduction: MI350 multiplies FP4 natively): the activations are
    quantized to MXFP4 by the quantizer above (alpha 1), then
    Y = dequant(quantize(A)) . dequant(W)^T and B = |.| . |.|^T in float64,
    with MXFP4 weights.  Returns (y_ref, bound)."""
    from .fp4_oracle import dequant_weights
    qc, qs = quantize_reference(a_bits, 1, 1.0)
    a = dequant_weights(qc, qs, K, 1)
    w = dequant_weights(codes, scales, K, 1)
    return a @ w.T, np.abs(a) @ np.abs(w).T
