"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each pin is independent of the oracle's code path: the E2M1 value list printed
on the mhpq.cn FP4 GEMM article (section 2.1), library FP8 decoders, exact
rational arithmetic, math.fsum brute force, closed forms and hand-worked
examples.  The mutation tests at the end plant plausible mistakes in the
oracle (on the CPU) and check that at least one pin fails for each.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import fp4_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- pin helpers
# Each helper raises AssertionError when the oracle module ``o`` is wrong.

def pin_e2m1_page_list(o):
    g = _golden("e2m1_value_list.json")
    vals = [float(o.e2m1_value(c)) for c in range(16)]
    assert vals[0] == 0.0
    assert sorted(vals[1:8]) == g["positive_nonzero_values"]
    assert vals[1:8] == g["positive_nonzero_values"], "E2M1 codes 1..7 must increase"
    for c in range(8):
        assert vals[c | 8] == -vals[c], "sign bit is bit 3"
    assert math.copysign(1.0, vals[8]) == -1.0, "code 8 is negative zero"
    states = {(v, math.copysign(1.0, v)) for v in vals}
    assert len(states) == g["total_states"]


def pin_e4m3_library(o):
    b = np.arange(256)
    ref = torch.from_numpy(b.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = o.e4m3_value(b)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def pin_e8m0_library(o):
    b = np.arange(256)
    ref = torch.from_numpy(b.astype(np.uint8)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = o.e8m0_value(b)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def _page_e2m1_fraction(code):
    """E2M1 value as an exact Fraction from the page's value list."""
    pos = [Fraction(0)] + [Fraction(v).limit_denominator(4)
                           for v in _golden("e2m1_value_list.json")["positive_nonzero_values"]]
    v = pos[code & 7]
    return -v if code & 8 else v


def _lib_scale_fraction(byte, fmt):
    t = torch.tensor([byte], dtype=torch.uint8)
    dt = torch.float8_e4m3fn if fmt == 0 else torch.float8_e8m0fnu
    return Fraction(float(t.view(dt).to(torch.float64)[0]))


def _codes_from_packed(packed, K):
    out = []
    for row in packed:
        r = []
        for byte in row:
            r += [byte & 15, byte >> 4]
        out.append(r[:K])
    return out


def pin_dequant_bruteforce(o):
    rng = np.random.Generator(np.random.PCG64(7))
    for fmt, K in ((0, 64), (1, 96)):
        G = 16 if fmt == 0 else 32
        N = 3
        codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        if fmt == 0:
            scales = rng.integers(0, 0x7F, size=(N, K // G), dtype=np.uint8)   # positive finite E4M3
        else:
            scales = rng.integers(100, 150, size=(N, K // G), dtype=np.uint8)
        got = o.dequant_weights(codes, scales, K, fmt)
        unpacked = _codes_from_packed(codes.tolist(), K)
        for n in range(N):
            for k in range(K):
                want = _page_e2m1_fraction(unpacked[n][k]) * _lib_scale_fraction(int(scales[n][k // G]), fmt)
                assert Fraction(float(got[n, k])) == want, (fmt, n, k)


def _bruteforce_gemm(a_rows, codes, scale_bytes, K, fmt):
    G = 16 if fmt == 0 else 32
    y, b = [], []
    for a in a_rows:
        yr, br = [], []
        for n in range(len(codes)):
            terms = [Fraction(a[k]) * _page_e2m1_fraction(codes[n][k])
                     * _lib_scale_fraction(scale_bytes[n][k // G], fmt) for k in range(K)]
            yr.append(sum(terms, Fraction(0)))
            br.append(sum((abs(t) for t in terms), Fraction(0)))
        y.append(yr)
        b.append(br)
    return y, b


def _a_bits(rows):
    return torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def pin_worked_examples(o):
    ex = _golden("worked_examples.json")
    # Hand-derived results (exact; see the derivations in the test docstrings).
    expected = {
        "nvfp4_2x16": ([[54.0, 2.8125], [0.0, 24.375]], [[54.0, 15.9375], [108.0, 31.875]]),
        "mxfp4_1x32": ([[19.0]], [[37.0]]),
    }
    for key, (y_hand, b_hand) in expected.items():
        e = ex[key]
        packed = np.array(e["packed_bytes"], dtype=np.uint8)
        assert _codes_from_packed(e["packed_bytes"], e["K"]) == e["codes"]
        scales = np.array(e["scale_bytes"], dtype=np.uint8)
        y, b = o.gemm_reference(_a_bits(e["A"]), packed, scales, e["K"], e["fmt"])
        assert y.tolist() == y_hand, key
        assert b.tolist() == b_hand, key
        yb, bb = _bruteforce_gemm(e["A"], e["codes"], e["scale_bytes"], e["K"], e["fmt"])
        assert [[float(v) for v in r] for r in yb] == y_hand
        assert [[float(v) for v in r] for r in bb] == b_hand


def pin_gemm_fsum(o):
    rng = np.random.Generator(np.random.PCG64(11))
    for fmt, (m, N, K) in ((0, (3, 5, 64)), (1, (2, 4, 128))):
        G = 16 if fmt == 0 else 32
        codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        scales = (rng.integers(0x20, 0x48, size=(N, K // G)) if fmt == 0
                  else rng.integers(120, 132, size=(N, K // G))).astype(np.uint8)
        a = rng.standard_normal((m, K)).astype(np.float32)
        a_bits = _a_bits(a.tolist())
        a_vals = torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        y, b = o.gemm_reference(a_bits, codes, scales, K, fmt)
        unpacked = _codes_from_packed(codes.tolist(), K)
        for i in range(m):
            for n in range(N):
                terms = [float(a_vals[i, k]) * float(_page_e2m1_fraction(unpacked[n][k]))
                         * float(_lib_scale_fraction(int(scales[n][k // G]), fmt)) for k in range(K)]
                s = math.fsum(terms)
                bb = math.fsum(abs(t) for t in terms)
                assert abs(y[i, n] - s) <= 1e-12 * bb, (fmt, i, n)
                assert abs(b[i, n] - bb) <= 1e-12 * bb


def pin_multi_group_scales(o):
    """Two groups with different scales: y = s0*sum(group 0) + s1*sum(group 1).

    K = 32, NVFP4: codes all 2 (value 1.0); group 0 scale 0x38 = 1.0, group 1
    scale 0x48 = 4.0; A row = [1]*16 ++ [0]*16 gives 16, [0]*16 ++ [1]*16 gives
    64, and A = k-th unit vector for k = 20 gives 4.
    """
    K = 32
    codes = np.full((1, K // 2), 0x22, dtype=np.uint8)
    scales = np.array([[0x38, 0x48]], dtype=np.uint8)
    rows = [[1.0] * 16 + [0.0] * 16, [0.0] * 16 + [1.0] * 16, [0.0] * K]
    rows[2][20] = 1.0
    y, _ = o.gemm_reference(_a_bits(rows), codes, scales, K, 0)
    assert y[:, 0].tolist() == [16.0, 64.0, 4.0]


def pin_nibble_order(o):
    """Byte 0x71 holds element 0 = code 1 (0.5) and element 1 = code 7 (6.0)."""
    codes = np.zeros((1, 8), dtype=np.uint8)
    codes[0, 0] = 0x71
    w = o.dequant_weights(codes, np.array([[0x38]], dtype=np.uint8), 16, 0)
    assert w[0, 0] == 0.5 and w[0, 1] == 6.0 and not np.any(w[0, 2:])


def pin_products_exact_in_bf16(o):
    """Closed form: an E2M1 value has <= 2 significant bits and an E4M3 scale
    <= 4, so code x scale has <= 6 significant bits; its exponent stays within
    [2^-10, 2688] for finite positive E4M3 and within the BF16 normal range for
    E8M0 exponents -125..125.  BF16 keeps 8 significant bits, so every product
    is exact: the oracle's dequantized values must convert without change."""
    codes = np.array([[c | (c << 4) for c in (0, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15)]],
                     dtype=np.uint8)
    K = 2 * codes.shape[1]                      # 30 elements, pad to a group multiple
    for fmt, scale_bytes in ((0, [b for b in range(0x7F)]), (1, list(range(2, 253)))):
        G = 16 if fmt == 0 else 32
        Kp = ((K + G - 1) // G) * G
        c = np.zeros((len(scale_bytes), Kp // 2), dtype=np.uint8)
        c[:, :codes.shape[1]] = codes
        s = np.repeat(np.array(scale_bytes, dtype=np.uint8)[:, None], Kp // G, axis=1)
        w = o.dequant_weights(c, s, Kp, fmt)
        bits = o.bf16_bits_of_exact(w)        # raises if any product is inexact
        back = o.bf16_bits_to_f64(bits)
        assert np.array_equal(back, w)
        for v in np.unique(np.abs(w[w != 0])):
            fr = Fraction(float(v))
            num = fr.numerator
            while num % 2 == 0:
                num //= 2
            assert num.bit_length() <= 6


def pin_tolerance(o):
    y_ref = np.array([[1.0, -3.0, 100.0, 0.0]])
    bound = np.array([[1.0, 3.0, 100.0, 50.0]])
    exact = _a_bits(y_ref.tolist())
    assert o.check_tolerance(exact, y_ref, bound).all()
    # beyond 8e-3 |y| + 2e-3 B
    bad = _a_bits([[1.0 + 0.02, -3.0 * 1.02, 100.0 * 1.02, 0.2]])
    assert not o.check_tolerance(bad, y_ref, bound).any()
    nan = _a_bits([[float("nan"), float("inf"), 100.0, 0.0]])
    assert o.check_tolerance(nan, y_ref, bound).tolist() == [[False, False, True, True]]


def pin_fp16_decode_library(o):
    """Every FP16 bit pattern decodes as the library's IEEE binary16 type."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = b.view(np.float16).astype(np.float64)
    got = o.fp16_bits_to_f64(b)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))
    assert np.array_equal(o.fp16_bits_of_exact(ref[ok]), b[ok])
    with pytest.raises(ValueError):
        o.fp16_bits_of_exact(np.array([1.0 + 2.0 ** -11]))


def _all_products(o, fmt, scale_bytes):
    codes = np.array([[c | (c << 4) for c in range(16)]], dtype=np.uint8)   # 32 elements
    G = 16 if fmt == 0 else 32
    c = np.repeat(codes, len(scale_bytes), axis=0)
    s = np.repeat(np.array(scale_bytes, dtype=np.uint8)[:, None], 32 // G, axis=1)
    return o.dequant_weights(c, s, 32, fmt)


def pin_products_exact_in_fp16(o):
    """Closed form for the FP16 variant: code x scale has <= 6 significant
    bits (FP16 keeps 11).  NVFP4: |product| lies in [2^-10, 2688] for every
    finite positive E4M3 scale, inside FP16's normal range, so every product
    is exact.  MXFP4: a nonzero product is 2^e times 0.5 .. 6 (a multiple of
    2^(e-1)); it is exact in FP16 iff 2^(e-1) >= 2^-24 (the smallest
    subnormal) and 6 x 2^e <= 65504, i.e. e in [-23, 13] (E8M0 bytes 104 ..
    140).  Bytes 103 and 141 must each hold an inexact product."""
    w = _all_products(o, 0, list(range(0x7F)))
    assert np.array_equal(o.fp16_bits_to_f64(o.fp16_bits_of_exact(w)), w)
    w = _all_products(o, 1, list(range(104, 141)))
    assert np.array_equal(o.fp16_bits_to_f64(o.fp16_bits_of_exact(w)), w)
    for byte in (103, 141):
        with pytest.raises(ValueError):
            o.fp16_bits_of_exact(_all_products(o, 1, [byte]))


def _f16_bits(rows):
    return np.asarray(rows, dtype=np.float64).astype(np.float16).view(np.uint16)


def pin_worked_examples_fp16(o):
    """The worked examples' activations are small integers, exact in FP16:
    with FP16 activation bits the reference must give the same hand-derived
    results as with BF16 bits."""
    ex = _golden("worked_examples.json")
    expected = {
        "nvfp4_2x16": ([[54.0, 2.8125], [0.0, 24.375]], [[54.0, 15.9375], [108.0, 31.875]]),
        "mxfp4_1x32": ([[19.0]], [[37.0]]),
    }
    for key, (y_hand, b_hand) in expected.items():
        e = ex[key]
        y, b = o.gemm_reference(_f16_bits(e["A"]), np.array(e["packed_bytes"], dtype=np.uint8),
                                np.array(e["scale_bytes"], dtype=np.uint8), e["K"], e["fmt"], act="f16")
        assert y.tolist() == y_hand, key
        assert b.tolist() == b_hand, key
        assert o.check_tolerance(_f16_bits(y_hand), y, b, act="f16").all()


def pin_tolerance_fp16(o):
    y_ref = np.array([[1.0, -3.0, 100.0, 0.0]])
    bound = np.array([[1.0, 3.0, 100.0, 50.0]])
    assert o.check_tolerance(_f16_bits(y_ref), y_ref, bound, act="f16").all()
    bad = _f16_bits([[1.02, -3.06, 102.0, 0.2]])
    assert not o.check_tolerance(bad, y_ref, bound, act="f16").any()
    # 65520 rounds to Inf in FP16: an overflowed output fails.
    assert not o.check_tolerance(_f16_bits([[65520.0]]), np.array([[65000.0]]),
                                 np.array([[65000.0]]), act="f16").any()


ALL_PINS = [pin_e2m1_page_list, pin_e4m3_library, pin_e8m0_library, pin_dequant_bruteforce,
            pin_worked_examples, pin_gemm_fsum, pin_multi_group_scales, pin_nibble_order,
            pin_products_exact_in_bf16, pin_tolerance, pin_fp16_decode_library,
            pin_products_exact_in_fp16, pin_worked_examples_fp16, pin_tolerance_fp16]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(O)


def test_scale_spot_values():
    v = O.e4m3_value(np.array([0x3C, 0x2A, 0x18, 0x48, 0x7E, 0x01, 0x38, 0x00]))
    assert v.tolist() == [1.5, 0.3125, 1 / 16, 4.0, 448.0, 2.0 ** -9, 1.0, 0.0]
    assert O.e8m0_value(np.array([127, 126, 129, 0])).tolist() == [1.0, 0.5, 4.0, 2.0 ** -127]
    assert np.isnan(O.e4m3_value(0x7F)) and np.isnan(O.e4m3_value(0xFF)) and np.isnan(O.e8m0_value(255))


def test_group_size_and_errors():
    assert O.group_size(0) == 16 and O.group_size(1) == 32
    with pytest.raises(ValueError):
        O.group_size(2)
    with pytest.raises(ValueError):
        O.dequant_weights(np.zeros((1, 12), np.uint8), np.zeros((1, 1), np.uint8), 24, 0)


# --------------------------------------------------------- planted mistakes
def _runs_clean(mod):
    failures = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError) as e:  # noqa: PERF203
            failures.append((pin.__name__, str(e)[:80]))
    return failures


class _Mutant:
    """The oracle module with one function replaced."""

    def __init__(self, **over):
        self._over = over

    def __getattr__(self, name):
        if name in self._over:
            return self._over[name]
        return getattr(O, name)


_ORIG_UNPACK = O.unpack_codes
_ORIG_E4M3 = O.e4m3_value
_ORIG_E2M1 = O.e2m1_value
_ORIG_FP16 = O.fp16_bits_to_f64


def _mut_e2m1_bias2(code):
    c = np.asarray(code, dtype=np.int64)
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = np.where(e == 0, m * 0.25, (1 + m / 2) * np.exp2(e - 2.0))
    return np.where(s == 1, -mag, mag)


def _mut_unpack_swapped(codes, K):
    out = _ORIG_UNPACK(codes, K)
    return out.reshape(out.shape[0], -1, 2)[:, :, ::-1].reshape(out.shape)


def _mut_e4m3_bias8(byte):
    return _ORIG_E4M3(byte) / 2.0


def _mut_dequant_group_shift(codes, scales, K, fmt):
    G = O.group_size(fmt)
    vals = O.e2m1_value(O.unpack_codes(codes, K))
    s = O.scale_value(scales, fmt)
    s = np.roll(np.repeat(s, G, axis=1), 1, axis=1)      # off-by-one group index
    return vals * s


def _mut_gemm_transposed(a_bits, codes, scales, K, fmt, act="bf16"):
    y, b = O.gemm_reference(a_bits, codes, scales, K, fmt, act)
    if y.shape[0] == y.shape[1]:
        return y.T, b.T
    return y, b


def _mut_gemm_no_abs_bound(a_bits, codes, scales, K, fmt, act="bf16"):
    a = O.act_bits_to_f64(a_bits, act)
    w = O.dequant_weights(codes, scales, K, fmt)
    return a @ w.T, np.abs(a @ w.T)


def _mut_fp16_bias16(bits):
    return _ORIG_FP16(bits) / 2.0


def _mut_gemm_act_ignored(a_bits, codes, scales, K, fmt, act="bf16"):
    return O.gemm_reference(a_bits, codes, scales, K, fmt)


def _mut_sign_dropped(code):
    return np.abs(_ORIG_E2M1(code))


@pytest.mark.parametrize("name,over", [
    ("e2m1 bias 2", {"e2m1_value": _mut_e2m1_bias2}),
    ("e2m1 sign dropped", {"e2m1_value": _mut_sign_dropped}),
    ("nibble order swapped", {"unpack_codes": _mut_unpack_swapped}),
    ("e4m3 read with bias 8", {"e4m3_value": _mut_e4m3_bias8}),
    ("scale group off by one", {"dequant_weights": _mut_dequant_group_shift}),
    ("output transposed", {"gemm_reference": _mut_gemm_transposed}),
    ("bound without abs", {"gemm_reference": _mut_gemm_no_abs_bound}),
    ("fp16 read with bias 16", {"fp16_bits_to_f64": _mut_fp16_bias16}),
    ("fp16 activations read as bf16", {"gemm_reference": _mut_gemm_act_ignored}),
])
def test_planted_mistake_is_caught(name, over):
    # The mutant module re-routes the named function; functions of the real
    # module that call it internally still use the original, so the mutants
    # are rebuilt on top of module-level replacements where needed.
    mod = _Mutant(**over)
    if {"e2m1_value", "unpack_codes", "e4m3_value", "fp16_bits_to_f64"} & set(over):
        saved = {k: getattr(O, k) for k in over}
        try:
            for k, v in over.items():
                setattr(O, k, v)
            failures = _runs_clean(O)
        finally:
            for k, v in saved.items():
                setattr(O, k, v)
    else:
        failures = _runs_clean(mod)
    assert failures, f"planted mistake '{name}' passed every pin"
    assert not _runs_clean(O), "the real oracle must pass every pin"


def test_package_exports():
    assert oracle.gemm_reference is O.gemm_reference


def test_gemm_reference_chunks_cover_every_row():
    """The oracle dequantizes and multiplies the weight rows in chunks of
    GEMM_CHUNK_ROWS: columns on both sides of every chunk boundary and in
    the ragged last chunk equal the math.fsum brute force of their dot
    products."""
    rng = np.random.Generator(np.random.PCG64(12))
    m, K, fmt = 2, 32, 0
    N = 2 * O.GEMM_CHUNK_ROWS + 37
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x48, size=(N, K // 16)).astype(np.uint8)
    a_bits = _a_bits(rng.standard_normal((m, K)).astype(np.float32).tolist())
    a_vals = torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    y, b = O.gemm_reference(a_bits, codes, scales, K, fmt)
    assert y.shape == (m, N) and b.shape == (m, N)
    C = O.GEMM_CHUNK_ROWS
    cols = [0, 1, C - 1, C, C + 1, 2 * C - 1, 2 * C, N - 2, N - 1]
    unpacked = _codes_from_packed(codes[cols].tolist(), K)
    for ci, n in enumerate(cols):
        for i in range(m):
            terms = [float(a_vals[i, k]) * float(_page_e2m1_fraction(unpacked[ci][k]))
                     * float(_lib_scale_fraction(int(scales[n][k // 16]), fmt)) for k in range(K)]
            s, bb = math.fsum(terms), math.fsum(abs(t) for t in terms)
            assert abs(y[i, n] - s) <= 1e-12 * bb and abs(b[i, n] - bb) <= 1e-12 * bb, (i, n)
