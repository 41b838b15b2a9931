"""Seeded random sweep of fp4_gemm / fp4_gemm_f16 / fp4_gemm_ex shapes against
the full CPU oracle.

The shapes are drawn (one fixed seed) across every regime the dispatch
distinguishes: the decode kernel with 16-, 32- and 64-row activation blocks
(with and without a K split), the 64-row prefill tiles of wide layers at
33 <= m <= 64, the prefill kernel with and without a K split, and its
256-row tiles on wide layers at m > 128; ragged m, N
and K (K any multiple of the group size, so K tails inside a 512-K scale
block), both weight formats, both activation types and, for some cases, a
per-tensor alpha.  Every output is compared with oracle.gemm_reference (scaled
by alpha where given) under the GEMM tolerance.  Sizes are bounded so that
the float64 oracle finishes each random case in well under a second and each
256-row tile case in a few seconds.
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


def _draw_cases(seed=20261203, n=44, budget=1.5e8):
    """(m, N, K, fmt, act, alpha) tuples: n regime-stratified random shapes
    with m * N * K <= budget, then four wide 33 <= m <= 64 layers with small K."""
    rng = np.random.Generator(np.random.PCG64(seed))
    regimes = [(1, 16), (17, 32), (33, 64), (65, 320)]
    cases = []
    while len(cases) < n:
        lo, hi = regimes[len(cases) % len(regimes)]
        m = int(rng.integers(lo, hi + 1))
        fmt = int(rng.integers(0, 2))
        G = 16 if fmt == 0 else 32
        N = int(rng.integers(1, 3001))
        K = G * int(rng.integers(1, 5120 // G + 1))
        if m * N * K > budget:
            continue
        act = "bf16" if rng.random() < 0.6 else "f16"
        alpha = 1.0 if rng.random() < 0.75 else float(np.float32(rng.uniform(0.1, 4.0)))
        cases.append((m, N, K, fmt, act, alpha))
    for _ in range(4):  # >= 128 groups of 256 columns: the wide-layer 64-row prefill tiles
        m = int(rng.integers(33, 65))
        fmt = int(rng.integers(0, 2))
        G = 16 if fmt == 0 else 32
        cases.append((m, 32768 + int(rng.integers(0, 300)), G * int(rng.integers(1, 8)), fmt, "bf16", 1.0))
    return cases


CASES = _draw_cases()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# 256-row prefill tiles (gemm_prefill_tall): m > 128 on layers wide enough
# that 128-row tiles take a second round of workgroups; ragged m inside one
# and two 256-row tiles, a partial last group of n-tiles, K tails inside a
# 512-K scale block, and a K split (long K at m = 129).
TALL_CASES = [
    (256, 32768 + 16, 512, 0, "bf16", 1.0),
    (129, 40000, 1088, 1, "f16", 1.0),
    (255, 57344, 512, 0, "bf16", 2.5),
    (500, 30000, 528, 0, "bf16", 1.0),
    (200, 36000, 1024 + 32, 1, "bf16", 0.75),
    (129, 8192, 28672, 0, "bf16", 1.0),
]


@pytest.mark.parametrize("m,N,K,fmt,act,alpha", CASES)
def test_random_shape_full_oracle(m, N, K, fmt, act, alpha):
    _check("random", m, N, K, fmt, act, alpha)


@pytest.mark.parametrize("m,N,K,fmt,act,alpha", TALL_CASES)
def test_tall_prefill_full_oracle(m, N, K, fmt, act, alpha):
    _check("tall", m, N, K, fmt, act, alpha)


def _check(tag, m, N, K, fmt, act, alpha):
    seed = (m * 1000003 + N * 7919 + K * 31 + fmt) % (1 << 31)
    print("[case]", tag, m, N, K, fmt, act, alpha, flush=True)
    p = synth.make_random(m, N, K, fmt, seed=seed, act=act)
    wq, sq = F.upload(*F.repack(p.codes, p.scales, N, K, fmt))
    tdt = torch.bfloat16 if act == "bf16" else torch.float16
    A = torch.from_numpy(np.ascontiguousarray(p.a_bits).view(np.int16)).cuda().view(tdt)
    C = F.gemm(A, wq, sq, N, K, fmt, alpha=alpha)
    torch.cuda.synchronize()
    y_bits = _bits(C)
    y_ref, bound = oracle.gemm_reference(p.a_bits, p.codes, p.scales, K, fmt, act)
    if alpha != 1.0:
        y_ref, bound = oracle.scaled_gemm_reference(y_ref, bound, alpha)
    ok = oracle.check_tolerance(y_bits, y_ref, bound, act=act)
    if not ok.all():
        i, n = np.argwhere(~ok)[0]
        y = oracle.act_bits_to_f64(y_bits, act)
        pytest.fail(f"{int((~ok).sum())} of {ok.size} outputs out of tolerance; first at m={i}, n={n}: "
                    f"gpu={y[i, n]!r} ref={y_ref[i, n]!r} bound={bound[i, n]!r}")
