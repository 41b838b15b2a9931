"""fp4_gemm and fp4_dequant at the size limits the boundary accepts (include/fp4gemm.h: K <= 2^20,
N <= 2^24, and the bytes of A and Y, m rounded up to the kernel's row block,
below 2^31), against the CPU oracle.

- Largest K: whole problems against the full oracle (decode, prefill, both
  formats, a K tail inside the last 512-K block).
- Largest A: A just under 2^31 bytes.  Its rows are drawn from 100 distinct
  seeded rows, so the oracle computes 100 rows and every output row is held
  to the tolerance of its source row.
- Largest N: more than 4 GiB of packed codes, so tile offsets pass 2^31 and
  2^32 bytes, and for the prefill case Y just under 2^31 bytes.  The packed
  arrays are seeded random bytes made on the device (valid scale bytes only);
  into a sample of 16-row tile slots (the first, the last, those at the 2^31
  and 2^32 byte boundaries and random ones) go the packed bytes of
  host-drawn weights (fp4_repack of a 16-row problem fills exactly one slot:
  the packed layout stores each 16-row tile contiguously, as the layout test
  on the CPU pins).  The oracle checks those columns; every output must be
  finite.
"""

import numpy as np
import pytest

import oracle
from mixed_precision_bf16_amd import fp4gemm as F
from mixed_precision_bf16_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KMAX = 1 << 20
NMAX = 1 << 24


@pytest.fixture(scope="module", autouse=True)
def gfx950():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    if not name.startswith("gfx950"):
        pytest.skip(f"needs gfx950, found {name}")
    F.lib()
    yield
    torch.cuda.empty_cache()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _a_dev(a_bits, act):
    tdt = torch.bfloat16 if act == "bf16" else torch.float16
    return torch.from_numpy(np.ascontiguousarray(a_bits).view(np.int16)).cuda().view(tdt)


def _assert_close(y_bits, y_ref, bound, act, what):
    ok = oracle.check_tolerance(y_bits, y_ref, bound, act=act)
    if not ok.all():
        i, n = np.argwhere(~ok)[0]
        y = oracle.act_bits_to_f64(y_bits, act)
        pytest.fail(f"{what}: {int((~ok).sum())} of {ok.size} outputs out of tolerance; first at ({i}, {n}): "
                    f"gpu={y[i, n]!r} ref={y_ref[i, n]!r} bound={bound[i, n]!r}")


@pytest.mark.parametrize("m,N,K,fmt,act", [
    (16, 40, KMAX, 0, "bf16"),          # decode, K split
    (200, 40, KMAX, 1, "bf16"),         # prefill tiles, K split and reduce
    (48, 300, KMAX - 16, 0, "f16"),     # 33 <= m <= 64, K tail in the last 512-K block
    (7, 1000, KMAX - 32, 1, "bf16"),
])
def test_largest_k_full_oracle(m, N, K, fmt, act):
    print("[case] largest K", m, N, K, fmt, act, flush=True)
    p = synth.make_random(m, N, K, fmt, seed=41 + m + N + fmt, act=act)
    wq, sq = F.upload(*F.repack(p.codes, p.scales, N, K, fmt))
    C = F.gemm(_a_dev(p.a_bits, act), wq, sq, N, K, fmt)
    torch.cuda.synchronize()
    y_ref, bound = oracle.gemm_reference(p.a_bits, p.codes, p.scales, K, fmt, act)
    _assert_close(_bits(C), y_ref, bound, act, "largest K")


@pytest.mark.parametrize("m,N,K,fmt,act", [
    (1000, 40, KMAX - 512, 0, "bf16"),  # 1024 x 1048064 x 2 B = 2^31 - 1 MiB after rounding m to 128
    (1023, 24, KMAX - 512, 1, "f16"),
])
def test_largest_a_rows_from_distinct_pool(m, N, K, fmt, act):
    assert -(-m // 128) * 128 * K * 2 < (1 << 31) <= -(-m // 128) * 128 * (K + 512) * 2
    print("[case] largest A", m, N, K, fmt, act, flush=True)
    pool = synth.make_random(100, N, K, fmt, seed=7 + m + fmt, act=act)
    src = np.random.Generator(np.random.PCG64(m)).integers(0, 100, size=m)
    wq, sq = F.upload(*F.repack(pool.codes, pool.scales, N, K, fmt))
    A = _a_dev(pool.a_bits[src], act)
    C = F.gemm(A, wq, sq, N, K, fmt)
    torch.cuda.synchronize()
    y_ref, bound = oracle.gemm_reference(pool.a_bits, pool.codes, pool.scales, K, fmt, act)
    _assert_close(_bits(C), y_ref[src], bound[src], act, "largest A")


def _sample_tiles(NT, tile_bytes, rng, extra=24):
    tiles = {0, 1, NT - 2, NT - 1}
    for edge in (1 << 31, 1 << 32):
        t = edge // tile_bytes
        tiles.update(x for x in (t - 1, t, t + 1) if 0 <= x < NT)
    tiles.update(int(x) for x in rng.choice(NT, size=min(extra, NT), replace=False))
    return sorted(t for t in tiles if 0 <= t < NT)


def _weights_with_sampled_tiles(N, K, fmt, seed):
    """Packed weights on the device: seeded random bytes (valid scale bytes
    only) with host-drawn 16-row tiles repacked into the sampled slots.
    Returns (wq, sq, codes, scales, cols): the host codes and scales of the
    sampled rows and their column (row of W) indices."""
    G = 16 if fmt == 0 else 32
    Kp = -(-K // 512) * 512
    NT = -(-N // 16)
    tile_codes, tile_scales = Kp * 8, (Kp // 512) * (512 if fmt == 0 else 256)
    wq_bytes, sq_bytes = F.repack_size(N, K, fmt)
    assert (wq_bytes, sq_bytes) == (NT * tile_codes, NT * tile_scales)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    wq = torch.randint(0, 256, (wq_bytes,), dtype=torch.uint8, device="cuda", generator=gen)
    lo, hi = (0x18, 0x48) if fmt == 0 else (127 - 6, 127 + 2)
    sq = torch.randint(lo, hi + 1, (sq_bytes,), dtype=torch.uint8, device="cuda", generator=gen)
    tiles = _sample_tiles(NT, tile_codes, np.random.Generator(np.random.PCG64(seed + N)))
    codes, scales, cols = [], [], []
    for i, t in enumerate(tiles):
        rows = min(16, N - 16 * t)
        tp = synth.make_random(1, rows, K, fmt, seed=5000 + 31 * i + seed)
        twq, tsq = F.repack(tp.codes, tp.scales, rows, K, fmt)
        assert twq.size == tile_codes and tsq.size == tile_scales
        wq[t * tile_codes:(t + 1) * tile_codes].copy_(torch.from_numpy(twq))
        sq[t * tile_scales:(t + 1) * tile_scales].copy_(torch.from_numpy(tsq))
        codes.append(tp.codes)
        scales.append(tp.scales)
        cols.append(16 * t + np.arange(rows))
    codes, scales, cols = np.concatenate(codes), np.concatenate(scales), np.concatenate(cols)
    assert scales.shape[1] == K // G
    print("[tiles]", tiles[:4], "..", tiles[-3:], flush=True)
    return wq, sq, codes, scales, cols


@pytest.mark.parametrize("m,N,K,fmt", [
    (16, NMAX, 1024, 0),                # decode, 8 GiB of codes
    (7, NMAX - 5, 512, 1),              # decode, ragged last tile
    (64, NMAX - 16, 512, 1),            # Y = 2^31 - 2 KiB
    (129, 8323056, 1024, 0),            # prefill 256-row tiles, Y just under 2^31 bytes, 4.3 GB of codes
])
def test_largest_n_sampled_tiles(m, N, K, fmt):
    assert N <= NMAX and m * N * 2 < (1 << 31)
    print("[case] largest N", m, N, K, fmt, flush=True)
    wq, sq, codes, scales, cols = _weights_with_sampled_tiles(N, K, fmt, 1000 + m)
    a_bits = synth.make_random(m, 1, K, fmt, seed=77 + m).a_bits
    C = F.gemm(_a_dev(a_bits, "bf16"), wq, sq, N, K, fmt)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(C).all())
    got = _bits(C.index_select(1, torch.from_numpy(cols).cuda()))
    del C, wq, sq
    torch.cuda.empty_cache()
    y_ref, bound = oracle.gemm_reference(a_bits, codes, scales, K, fmt)
    _assert_close(got, y_ref, bound, "bf16", "largest N")


@pytest.mark.parametrize("N,K,fmt", [(NMAX, 512, 0), (16, KMAX, 1), (40, KMAX - 16, 0)])
def test_dequant_at_the_limits_bit_exact(N, K, fmt):
    """fp4_dequant (the weights exactly as the GEMM feeds them to the matrix
    core) at the largest N (a 16 GiB output) and the largest K: the sampled
    rows bit-exact against the oracle's dequantized weights, every value
    finite."""
    print("[case] dequant at the limits", N, K, fmt, flush=True)
    wq, sq, codes, scales, cols = _weights_with_sampled_tiles(N, K, fmt, 2000 + fmt)
    W = F.dequant(wq, sq, N, K, fmt)
    torch.cuda.synchronize()
    del wq, sq
    assert bool(torch.isfinite(W).all())
    got = _bits(W.index_select(0, torch.from_numpy(cols).cuda()))
    del W
    torch.cuda.empty_cache()
    want = oracle.bf16_bits_of_exact(oracle.dequant_weights(codes, scales, K, fmt))
    nz = oracle.dequant_weights(codes, scales, K, fmt) != 0
    assert np.array_equal(got[nz], want[nz]), np.argwhere((got != want) & nz)[:5]
    assert not np.any(oracle.bf16_bits_to_f64(got)[~nz]), "zero weights dequantize to +-0"
