"""Pins of the quantizer oracle (oracle.quant_oracle) against facts outside it.

* E4M3 encoding: round-to-nearest-even bytes equal the library's FP32 ->
  float8_e4m3fn cast over random values and every exact midpoint.
* Nearest grid point: exact rational brute force over the E2M1 grid, ties to
  the even code, on random quotients and every midpoint.
* Fixed point: weights built as code x scale with a full-range block maximum
  quantize back to exactly those codes and scales (both formats).
* The zero-block rule (positive scale, zero codes), saturation, no negative
  zero, and the error bound |w - dequant| <= S * (half the local grid gap).
* MXFP4 blocks below 2^-124 (scale byte 0 = 2^-127): exact rational block
  scaling, and the fixed point at scale bytes 0, 1, 2.
Planted mistakes (ties away from zero, scale = amax, sign dropped, E8M0
exponent rounded up, E8M0 byte 0 flushing its block) each fail a pin.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp4_oracle as O
from oracle import quant_oracle as Q

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
        Fraction(6)]


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def pin_e4m3_encode_library(q):
    rng = np.random.Generator(np.random.PCG64(1))
    x = np.exp2(rng.uniform(-12, 8.8, size=4000)).astype(np.float32)
    vals = O.e4m3_value(np.arange(1, 0x7F)).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)            # exact in FP32
    x = np.concatenate([x, mids, vals.astype(np.float32)])
    x = x[x < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q.e4m3_rne_byte(x), ref)


def pin_nearest_grid_bruteforce(q):
    rng = np.random.Generator(np.random.PCG64(2))
    xs = list(rng.uniform(0, 7, size=300).astype(np.float32)) + \
        [float(GRID[i] + GRID[i + 1]) / 2 for i in range(7)] + [0.0, 6.0, 9.5]
    got = q.nearest_e2m1(np.array(xs, dtype=np.float32))
    for x, g in zip(xs, got):
        fx = Fraction(float(x))
        d = [abs(v - fx) for v in GRID]
        best = [i for i in range(8) if d[i] == min(d)]
        want = best[0] if len(best) == 1 else [i for i in best if i % 2 == 0][0]
        if fx > 6:
            want = 7
        assert g == want, (x, g, want)


def pin_fixed_point(q):
    rng = np.random.Generator(np.random.PCG64(3))
    for fmt in (0, 1):
        G = 16 if fmt == 0 else 32
        N, K = 6, 4 * G
        codes = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
        codes[codes == 8] = 0
        codes[:, ::G] = 7                                              # block maximum 6 x scale
        if fmt == 0:
            sb = rng.integers(0x08, 0x50, size=(N, K // G)).astype(np.uint8)   # normal E4M3
        else:
            sb = rng.integers(110, 140, size=(N, K // G)).astype(np.uint8)
            sb[0] = [0, 1, 2, 0]        # the smallest E8M0 scales: 2^-127 (byte 0), 2^-126, 2^-125
        packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        w = O.dequant_weights(packed, sb, K, fmt)
        c2, s2 = q.quantize_reference(O.bf16_bits_of_exact(w), fmt)
        assert np.array_equal(s2, sb), fmt
        assert np.array_equal(c2, packed), fmt


def pin_zero_block_and_signs(q):
    w = np.zeros((2, 32), np.float32)
    w[1, :16] = -1e-30                                                 # rounds to code 0: no negative zero
    w[1, 16:] = [-6.0, 100.0] + [0.0] * 14
    for fmt in (0, 1):
        c, s = q.quantize_reference(_bf16_bits(w), fmt)
        codes = O.unpack_codes(c, 32)
        assert not np.any(codes == 8)
        assert not np.any(codes[0]) and not np.any(codes[1, :16])
        if fmt == 0:
            assert s[0].tolist() == [1, 1]                             # positive floor, not zero
        else:
            assert s[0].tolist() == [0]
        assert codes[1, 17] == 7                                       # block maximum -> 6


def pin_error_bound(q):
    rng = np.random.Generator(np.random.PCG64(4))
    for fmt in (0, 1):
        G = 16 if fmt == 0 else 32
        w = (rng.standard_normal((8, 8 * G)) * np.exp2(rng.uniform(-6, 4, size=(8, 1)))).astype(np.float32)
        bits = _bf16_bits(w)
        x = O.bf16_bits_to_f64(bits)
        c, s = q.quantize_reference(bits, fmt)
        d = O.dequant_weights(c, s, 8 * G, fmt)
        S = np.repeat(O.scale_value(s, fmt), G, axis=1)
        qq = np.abs(x) / S
        half_gap = np.where(qq < 2, 0.25, np.where(qq < 4, 0.5, 1.0))
        sat = qq > 6
        assert np.all(np.abs(d - x)[~sat] <= S[~sat] * half_gap[~sat] * (1 + 1e-6))
        assert np.all(np.abs(d[sat]) == 6 * S[sat])


def _frac_floor_log2(x: Fraction) -> int:
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def pin_tiny_mx_blocks_exact(q):
    """MXFP4 blocks whose maximum lies below 2^-124 (scale byte 0 = 2^-127):
    exact rational arithmetic of block scaling (divide by the block's scale,
    then round to the nearest grid value, ties to the even code, saturating
    at 6; mhpq.cn article sections 2.1 and 2.2) with the scale
    2^max(floor(log2 amax) - 2, -127).  A non-zero element that does not
    round to zero keeps a non-zero code."""
    amaxes = [2.0 ** -126, 1.5 * 2.0 ** -125, 1.8984375 * 2.0 ** -125, 2.0 ** -124, 1.75 * 2.0 ** -127]
    rng = np.random.Generator(np.random.PCG64(5))
    w = np.zeros((len(amaxes), 32), np.float32)
    for i, a in enumerate(amaxes):
        w[i, 0] = a
        w[i, 1:] = (rng.uniform(-1, 1, size=31) * a).astype(np.float32)
        w[i, 1:4] = [-a / 2, a / 3, 2.0 ** -133]            # a midpoint-ish value and the smallest BF16
    bits = _bf16_bits(w)
    x = O.bf16_bits_to_f64(bits)
    c, s = q.quantize_reference(bits, 1)
    codes = O.unpack_codes(c, 32)
    for i in range(len(amaxes)):
        fr = [Fraction(float(v)) for v in x[i]]
        amax = max(abs(v) for v in fr)
        e = max(_frac_floor_log2(amax) - 2, -127)
        assert int(s[i, 0]) == e + 127, (i, s[i, 0], e)
        S = Fraction(2) ** e
        for k, v in enumerate(fr):
            qv = abs(v) / S
            d = [abs(g - qv) for g in GRID]
            best = [j for j in range(8) if d[j] == min(d)]
            mag = best[0] if len(best) == 1 else [j for j in best if j % 2 == 0][0]
            if qv > 6:
                mag = 7
            want = mag | (8 if (v < 0 and mag) else 0)
            assert codes[i, k] == want, (i, k, float(v), codes[i, k], want)
    assert np.all(codes[:, 0] != 0), "each block maximum keeps a non-zero code"


ALL_PINS = [pin_e4m3_encode_library, pin_nearest_grid_bruteforce, pin_fixed_point, pin_zero_block_and_signs,
            pin_error_bound, pin_tiny_mx_blocks_exact]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_quant_oracle_pin(pin):
    pin(Q)


def test_alpha_scales_output_and_scales():
    y, b = np.array([[1.0, -2.0]]), np.array([[3.0, 4.0]])
    y2, b2 = Q.scaled_gemm_reference(y, b, 0.25)
    assert y2.tolist() == [[0.25, -0.5]] and b2.tolist() == [[0.75, 1.0]]
    w = _bf16_bits(np.linspace(-3, 3, 64, dtype=np.float32).reshape(2, 32))
    c1, s1 = Q.quantize_reference(w, 0, alpha=1.0)
    c2, s2 = Q.quantize_reference(w, 0, alpha=0.5)       # scales double, codes unchanged
    assert np.array_equal(c1, c2)
    assert np.array_equal(O.e4m3_value(s2), 2 * O.e4m3_value(s1))


def test_native_reference_equals_dense_on_representable_activations():
    """Activations that are exact MXFP4 values (code x 2^e with a full-range
    block maximum) quantize to themselves (the fixed-point pin), so the
    native reference must equal the pinned dense reference exactly; on
    general activations it must differ (it quantizes)."""
    rng = np.random.Generator(np.random.PCG64(6))
    m, N, K = 5, 7, 128
    acodes = rng.integers(0, 16, size=(m, K)).astype(np.uint8)
    acodes[acodes == 8] = 0
    acodes[:, ::32] = 7
    apacked = (acodes[:, 0::2] | (acodes[:, 1::2] << 4)).astype(np.uint8)
    ascales = rng.integers(120, 134, size=(m, K // 32)).astype(np.uint8)
    a_bits = O.bf16_bits_of_exact(O.dequant_weights(apacked, ascales, K, 1))
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(120, 134, size=(N, K // 32)).astype(np.uint8)
    y, b = O.gemm_reference(a_bits, codes, scales, K, 1)
    yn, bn = Q.native_reference(a_bits, codes, scales, K)
    assert np.array_equal(y, yn) and np.array_equal(b, bn)
    g = _bf16_bits(rng.standard_normal((m, K)).astype(np.float32))
    y, _ = O.gemm_reference(g, codes, scales, K, 1)
    yn, _ = Q.native_reference(g, codes, scales, K)
    assert not np.array_equal(y, yn)


class _Mut:
    def __init__(self, **over):
        self.__dict__.update({k: getattr(Q, k) for k in ("e4m3_rne_byte", "nearest_e2m1", "quantize_reference")})
        self.__dict__.update(over)


def _mut_ties_away(qv):
    qv = np.asarray(qv, dtype=np.float64)
    g = Q.GRID
    out = Q.nearest_e2m1(qv)
    for i in range(7):
        mid = (g[i] + g[i + 1]) / 2
        out = np.where(qv == mid, i + 1, out)
    return out


def _mut_scale_amax(w_bits, fmt, alpha=1.0):
    w = O.bf16_bits_to_f64(w_bits) / 6.0
    return Q.quantize_reference(O.bf16_bits_of_exact(np.round(w * 256) / 256), fmt, alpha)


def _mut_no_sign(w_bits, fmt, alpha=1.0):
    c, s = Q.quantize_reference(w_bits, fmt, alpha)
    return (c & 0x77).astype(np.uint8), s


def _mut_e8m0_ceil(w_bits, fmt, alpha=1.0):
    c, s = Q.quantize_reference(w_bits, fmt, alpha)
    if fmt == 1:
        s = np.minimum(s.astype(np.int64) + 1, 254).astype(np.uint8)
    return c, s


def _mut_byte0_flush(w_bits, fmt, alpha=1.0):
    # a reading that zeroes every code of a block whose E8M0 scale byte is 0
    c, s = Q.quantize_reference(w_bits, fmt, alpha)
    if fmt == 1:
        K = c.shape[1] * 2
        blk = np.repeat(s == 0, 16, axis=1)
        c = np.where(blk, 0, c).astype(np.uint8)
        assert c.shape[1] * 2 == K
    return c, s


@pytest.mark.parametrize("name,over", [
    ("ties away from zero", {"nearest_e2m1": _mut_ties_away}),
    ("E8M0 byte 0 flushes its block", {"quantize_reference": _mut_byte0_flush}),
    ("scale = amax", {"quantize_reference": _mut_scale_amax}),
    ("sign dropped", {"quantize_reference": _mut_no_sign}),
    ("E8M0 exponent rounded up", {"quantize_reference": _mut_e8m0_ceil}),
])
def test_planted_mistake_is_caught(name, over):
    failures = 0
    for pin in ALL_PINS:
        try:
            pin(_Mut(**over))
        except (AssertionError, ValueError):
            failures += 1
    assert failures, f"planted mistake '{name}' passed every pin"
