"""GPU parity of the offline quantizer (fp4_quantize) and of the per-tensor
output scale (fp4_gemm_ex), through the C ABI, against the CPU oracle.

Bars: quantizer codes and scale bytes bit-exact against
oracle.quantize_reference (integer output decided in FP32 on both sides);
fp4_gemm_ex with alpha = 2^-3 bit-identical to fp4_gemm's output scaled by
2^-3, and any alpha within alpha x the GEMM tolerance of the oracle.
"""

import numpy as np
import pytest

import oracle
from mixed_precision_bf16_amd import fp4gemm as F
from mixed_precision_bf16_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    if not name.startswith("gfx950"):
        pytest.skip(f"needs gfx950, found {name}")
    F.lib()
    yield


def _say(*a):
    print("[case]", *a, flush=True)


def _weights(N, K, fmt, seed, specials=True):
    """BF16 weight bits: N(0,1) times a per-row power of two in 2^-8 .. 2^8,
    plus (specials) zero blocks, exact grid midpoints, NaN, +-Inf and
    negative values that round to zero."""
    rng = np.random.Generator(np.random.PCG64(seed))
    G = 16 if fmt == 0 else 32
    w = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-8, 9, size=(N, 1)))).astype(np.float32)
    if specials and N >= 4:
        w[0, :G] = 0.0                                             # zero block
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
        blk = np.zeros(G, np.float32)
        blk[0] = 6.0                                               # block max 6 -> scale 1
        blk[1:1 + 7] = mids
        blk[8:15] = -mids
        w[1, :G] = blk
        if K >= 4 * G:
            w[2, G:2 * G] = -1e-30
            w[2, 2 * G] = -7.0
            w[3, 3 * G] = np.nan
            w[3, 3 * G + 1] = 2.0
            w[3, 2 * G] = np.inf
            w[3, 2 * G + 1] = -np.inf
    bits = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bits


@pytest.mark.parametrize("fmt,N,K,alpha", [(0, 37, 512, 1.0), (1, 37, 512, 1.0), (0, 1000, 8192, 1.0),
                                           (1, 640, 2880, 1.0), (0, 64, 1024, 0.37), (1, 64, 1024, 2.0 ** -7),
                                           (0, 5, 16, 1.0), (1, 3, 32, 3.0)])
def test_quantize_bit_exact(fmt, N, K, alpha):
    bits = _weights(N, K, fmt, seed=N + K + fmt)
    _say("quantize", fmt, N, K, alpha)
    want_c, want_s = oracle.quantize_reference(bits, fmt, alpha)
    W = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    c, s = F.quantize(W, fmt, alpha)
    torch.cuda.synchronize()
    c, s = c.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(s, want_s), np.argwhere(s != want_s)[:5]
    assert np.array_equal(c, want_c), np.argwhere(c != want_c)[:5]


@pytest.mark.parametrize("fmt,N,K", [(0, 163877, 16384), (1, 260, 1 << 24)])
def test_quantize_many_launches_bit_exact(fmt, N, K):
    """More G-element blocks than one quantizer launch covers (the library
    launches at most 2^26 blocks, whole rows, at a time; here 2.5 and 2 such
    slices plus a ragged one, the second at the largest K).  The weights are
    seeded random BF16 made on the device; at the first and last row, at
    random rows and at the rows on both sides of each slice boundary, the
    first and last 4096 elements are replaced by host-drawn blocks (with the
    special values of _weights), whose codes and scales must match the oracle
    bit for bit."""
    G = 16 if fmt == 0 else 32
    SEG = 4096
    rows_per = (1 << 26) // (K // G)
    rows = {0, N - 1}
    for b in range(rows_per, N, rows_per):
        rows.update((b - 1, b))
    rows.update(int(x) for x in np.random.Generator(np.random.PCG64(N)).choice(N, 6, replace=False))
    rows = sorted(rows)
    _say("quantize, several launches", fmt, N, K, rows)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(N + fmt)
    W = torch.randn((N, K), dtype=torch.bfloat16, device="cuda", generator=gen)
    seg = _weights(2 * len(rows), SEG, fmt, seed=3 * N + fmt)
    for i, r in enumerate(rows):
        W[r, :SEG].copy_(torch.from_numpy(seg[2 * i].view(np.int16)).view(torch.bfloat16))
        W[r, K - SEG:].copy_(torch.from_numpy(seg[2 * i + 1].view(np.int16)).view(torch.bfloat16))
    c, s = F.quantize(W, fmt)
    torch.cuda.synchronize()
    del W
    idx = torch.tensor(rows, device="cuda")
    c, s = c.index_select(0, idx).cpu().numpy(), s.index_select(0, idx).cpu().numpy()
    torch.cuda.empty_cache()
    got_c = np.stack([c[:, :SEG // 2], c[:, K // 2 - SEG // 2:]], axis=1).reshape(2 * len(rows), SEG // 2)
    got_s = np.stack([s[:, :SEG // G], s[:, K // G - SEG // G:]], axis=1).reshape(2 * len(rows), SEG // G)
    want_c, want_s = oracle.quantize_reference(seg, fmt, 1.0)
    assert np.array_equal(got_s, want_s), np.argwhere(got_s != want_s)[:5]
    assert np.array_equal(got_c, want_c), np.argwhere(got_c != want_c)[:5]


def _midpoint_weights(N, K, fmt, alpha, seed):
    """BF16 weight bits whose every block has a chosen scale (an E4M3 value,
    or a power of two for MXFP4: the block maximum is 6 x scale x alpha) and
    whose other elements are E2M1 values and exact midpoints between them
    times that scale, a quarter of them moved to a BF16 neighbour: the cases
    where a decision by a rounded quotient would go wrong."""
    rng = np.random.Generator(np.random.PCG64(seed))
    G = 16 if fmt == 0 else 32
    nb = K // G
    vals = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    if fmt == 0:
        e4 = oracle.e4m3_value(np.arange(1, 0x7F))
        s = e4[rng.integers(0, len(e4), size=(N, nb))]
    else:
        s = np.exp2(rng.integers(-20, 20, size=(N, nb)).astype(np.float64))
    w = vals[rng.integers(0, len(vals), size=(N, nb, G))] * (s * alpha)[..., None]
    w[..., 0] = 6.0 * s * alpha
    w *= np.where(rng.random((N, nb, G)) < 0.5, -1.0, 1.0)
    bits = torch.from_numpy(w.astype(np.float32).reshape(N, K)).to(torch.bfloat16).view(torch.int16).numpy()
    bits = bits.view(np.uint16).copy()
    step = np.where(rng.random(bits.shape) < 0.5, 1, -1)
    nudge = rng.random(bits.shape) < 0.25
    return np.where(nudge, bits.astype(np.int64) + step, bits).astype(np.uint16)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("alpha", [1.0, 2.0 ** -7, 2.0 ** 20])
def test_quantize_midpoint_blocks_bit_exact(fmt, alpha):
    """With alpha a power of two the quantizer decides by the hardware FP32 ->
    FP4 convert (NVFP4: on x / M snapped to 3 significant bits near a
    midpoint); blocks made of exact midpoints and their neighbours under
    every scale meet the oracle's nearest-even rule bit for bit."""
    bits = _midpoint_weights(128, 1024, fmt, alpha, seed=31 + fmt)
    _say("quantize midpoints", fmt, alpha)
    want_c, want_s = oracle.quantize_reference(bits, fmt, alpha)
    W = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    c, s = F.quantize(W, fmt, alpha)
    torch.cuda.synchronize()
    c, s = c.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(s, want_s), np.argwhere(s != want_s)[:5]
    assert np.array_equal(c, want_c), np.argwhere(c != want_c)[:5]


@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_then_gemm_parity(fmt):
    """Device-quantized weights through repack and the GEMM: within the
    tolerance of the oracle's GEMM on the same codes and scales, and
    fp4_gemm_ex with the quantizer's alpha matches alpha x that."""
    N, K, m, alpha = 520, 2048, 16, 0.5 if fmt == 0 else 1.0
    bits = _weights(N, K, fmt, seed=11 + fmt, specials=False)
    _say("quantize -> gemm", fmt)
    W = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    c, s = F.quantize(W, fmt, alpha)
    codes, scales = c.cpu().numpy(), s.cpu().numpy()
    wq, sq = F.upload(*F.repack(codes, scales, N, K, fmt))
    p = synth.make_random(m, N, K, fmt, seed=3)
    A = torch.from_numpy(p.a_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y = F.gemm(A, wq, sq, N, K, fmt, alpha=alpha)
    torch.cuda.synchronize()
    y_ref, bound = oracle.gemm_reference(p.a_bits, codes, scales, K, fmt)
    y_ref, bound = oracle.scaled_gemm_reference(y_ref, bound, alpha)
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert oracle.check_tolerance(yb, y_ref, bound).all()
    # the quantized weights approximate W: |alpha x dequant - w| <= alpha x scale wherever |w| <= 6 alpha
    # x scale; elements beyond (the block maximum when the scale rounded down) saturate to 6 alpha x scale
    w = oracle.bf16_bits_to_f64(bits)
    d = alpha * oracle.dequant_weights(codes, scales, K, fmt)
    G = 16 if fmt == 0 else 32
    S = alpha * np.repeat(oracle.scale_value(scales, fmt), G, axis=1)
    inside = np.abs(w) <= 6 * S
    assert np.all((np.abs(d - w) <= S * (1 + 1e-6))[inside])
    assert np.all((np.abs(d) == 6 * S)[~inside])


@pytest.mark.parametrize("m,N,K,fmt,act", [(16, 8192, 8192, 0, 0), (16, 8192, 28672, 0, 0), (256, 1024, 4096, 0, 0),
                                           (100, 520, 2048, 1, 0), (16, 4096, 8192, 0, 1), (256, 512, 2048, 1, 1),
                                           (5, 40, 48, 0, 0)])
def test_gemm_ex_alpha(m, N, K, fmt, act):
    """alpha = 2^-3 is exact: bit-identical to the unscaled output times 2^-3
    (decode with and without a K split, prefill, both activation types);
    alpha = 0.3 within 0.3 x the tolerance of the oracle."""
    tdt = torch.bfloat16 if act == 0 else torch.float16
    p = synth.make_random(m, N, K, fmt, seed=m + N + K, act="bf16" if act == 0 else "f16")
    _say("gemm_ex", m, N, K, fmt, act)
    wq, sq = F.upload(*F.repack(p.codes, p.scales, N, K, fmt))
    A = torch.from_numpy(p.a_bits.view(np.int16)).cuda().view(tdt)
    y1 = F.gemm(A, wq, sq, N, K, fmt)
    y8 = F.gemm(A, wq, sq, N, K, fmt, alpha=0.125)
    y3 = F.gemm(A, wq, sq, N, K, fmt, alpha=0.3)
    torch.cuda.synchronize()
    assert torch.equal((y1.float() * 0.125).to(tdt), y8)
    yb = y3.view(torch.int16).cpu().numpy().view(np.uint16)
    rows = np.arange(N) if N <= 1024 else np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N),
                                                                    np.arange(0, N, 97)]))
    y_ref, bound = oracle.gemm_reference(p.a_bits, p.codes[rows], p.scales[rows], K, fmt, p.act)
    y_ref, bound = oracle.scaled_gemm_reference(y_ref, bound, 0.3)
    assert oracle.check_tolerance(yb[:, rows], y_ref, bound, act=p.act).all()


def tiny_mx_weights(N, seed):
    """BF16 weight bits [N][128] whose MXFP4 blocks have maxima below 2^-124
    (scale byte 0 = 2^-127, the FP32 subnormal on the device) or just above
    it, plus exact code x 2^-127 / 2^-126 / 2^-125 blocks (the fixed point of
    the quantizer at scale bytes 0, 1, 2) and the smallest BF16 subnormal."""
    rng = np.random.Generator(np.random.PCG64(seed))
    amax = np.array([2.0 ** -126, 1.5 * 2.0 ** -125, 1.8984375 * 2.0 ** -125, 2.0 ** -124, 1.75 * 2.0 ** -127,
                     2.0 ** -123])
    w = np.zeros((N, 128), np.float32)
    for i in range(N):
        for b in range(4):
            a = amax[(i + b) % len(amax)]
            blk = (rng.uniform(-1, 1, size=32) * a).astype(np.float32)
            blk[rng.integers(0, 32)] = a if (i + b) % 2 == 0 else -a
            blk[rng.integers(0, 32)] = 2.0 ** -133
            w[i, 32 * b:32 * b + 32] = blk
    ex = rng.integers(0, 16, size=(3, 128))
    ex[ex == 8] = 0
    ex[:, ::32] = 7
    vals = oracle.e2m1_value(ex) * np.exp2(np.array([-127.0, -126.0, -125.0]))[:, None]
    w[:3] = vals.astype(np.float32)
    return torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("alpha", [1.0, 2.0 ** -7, 0.37, 8.0])
def test_quantize_tiny_mxfp4_blocks_bit_exact(alpha):
    """Scale byte 0 is the scale 2^-127 and its block is rounded like any
    other (block scaling: divide by the block's scale, then round)."""
    bits = tiny_mx_weights(24, seed=77)
    _say("quantize tiny mxfp4", alpha)
    want_c, want_s = oracle.quantize_reference(bits, 1, alpha)
    if alpha == 1.0:
        assert np.any(want_s == 0) and np.any(want_c[want_s.repeat(16, axis=1) == 0] != 0)
    W = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    c, s = F.quantize(W, 1, alpha)
    torch.cuda.synchronize()
    c, s = c.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(s, want_s), np.argwhere(s != want_s)[:5]
    assert np.array_equal(c, want_c), np.argwhere(c != want_c)[:5]


def test_native_tiny_activation_blocks():
    """The native path quantizes its activations with the same rule: rows of
    A made of blocks below 2^-124 (scale byte 0) against MXFP4 weights with
    large scales (2^30 .. 2^40, so the products stay FP32 normals) meet
    oracle.native_reference."""
    m, N, K = 24, 96, 128
    a_bits = tiny_mx_weights(m, seed=78)
    p = synth.make_random(m, N, K, 1, seed=79, scale_lo=30, scale_hi=40)
    p = synth.Problem("native_tiny", m, N, K, 1, a_bits, p.codes, p.scales, 79)
    _say("native tiny activations")
    wq, sq = F.native_repack(p.codes, p.scales, N, K)
    A = torch.from_numpy(a_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y = F.gemm_native(A, wq.cuda(), sq.cuda(), N, K)
    torch.cuda.synchronize()
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    y_ref, bound = oracle.native_reference(a_bits, p.codes, p.scales, K)
    assert np.all(np.abs(y_ref).max(axis=1) > 0), "every row keeps non-zero quantized activations"
    assert oracle.check_tolerance(yb, y_ref, bound).all()

