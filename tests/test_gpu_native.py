"""GPU parity of the native FP4 path (fp4_gemm_native: activations quantized
to MXFP4 on the device, FP4 x FP4 on the gfx950 matrix cores) against the
CPU oracle (oracle.native_reference), through the C ABI.

Bar: |y - y_ref| <= 8e-3 |y_ref| + 2e-3 sum_k |a'_k w_k| element by element,
with a' the oracle's MXFP4 activations (the device quantizer's codes and
scales are bit-exact to the oracle's, tests/test_gpu_quant.py); on
activations that are exact MXFP4 values the path must also meet the dense
reference.  Full-size shapes on sampled output columns.
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


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_native(p, alpha=1.0, reps=1):
    wq, sq = F.native_repack(p.codes, p.scales, p.N, p.K)
    wq, sq = wq.cuda(), sq.cuda()
    A = torch.from_numpy(np.ascontiguousarray(p.a_bits).view(np.int16)).cuda().view(torch.bfloat16)
    outs = []
    for _ in range(reps):
        y = F.gemm_native(A, wq, sq, p.N, p.K, alpha=alpha)
        torch.cuda.synchronize()
        outs.append(_bits(y))
    return outs if reps > 1 else outs[0]


def check(p, y_bits, rows=None, alpha=1.0):
    codes, scales = (p.codes, p.scales) if rows is None else (p.codes[rows], p.scales[rows])
    y_ref, bound = oracle.native_reference(p.a_bits, codes, scales, p.K)
    y_ref, bound = oracle.scaled_gemm_reference(y_ref, bound, alpha)
    yb = y_bits if rows is None else y_bits[:, rows]
    ok = oracle.check_tolerance(yb, y_ref, bound)
    if not ok.all():
        i, n = np.argwhere(~ok)[0]
        y = oracle.bf16_bits_to_f64(yb)
        raise AssertionError(f"{p.name}: {int((~ok).sum())} of {ok.size} out of tolerance; first at m={i}, n={n}: "
                             f"gpu={y[i, n]!r} ref={y_ref[i, n]!r} bound={bound[i, n]!r}")


NATIVE = [(1, 16, 32), (5, 40, 64), (16, 100, 512), (33, 130, 2880), (64, 257, 1024), (100, 260, 1024),
          (256, 512, 2048), (300, 96, 640), (129, 1000, 4096)]


@pytest.mark.parametrize("m,N,K", NATIVE)
def test_native_full_oracle(m, N, K):
    p = synth.make_random(m, N, K, 1, seed=m * 31 + N + K)
    _say("native", m, N, K)
    check(p, run_native(p))


def test_native_alpha_and_exact_activations():
    """Activations that are exact MXFP4 values: the native result also meets
    the dense reference; alpha scales the output."""
    rng = np.random.Generator(np.random.PCG64(9))
    m, N, K = 48, 320, 1024
    ac = rng.integers(0, 16, size=(m, K)).astype(np.uint8)
    ac[ac == 8] = 0
    ac[:, ::32] = 7
    apacked = (ac[:, 0::2] | (ac[:, 1::2] << 4)).astype(np.uint8)
    ascales = rng.integers(122, 132, size=(m, K // 32)).astype(np.uint8)
    a_bits = oracle.bf16_bits_of_exact(oracle.dequant_weights(apacked, ascales, K, 1))
    p = synth.make_random(m, N, K, 1, seed=4)
    p = synth.Problem("native_exact", m, N, K, 1, a_bits, p.codes, p.scales, 4)
    _say("native exact activations")
    y = run_native(p)
    y_ref, bound = oracle.gemm_reference(a_bits, p.codes, p.scales, K, 1)
    assert oracle.check_tolerance(y, y_ref, bound).all()
    y2 = run_native(p, alpha=0.25)
    assert np.array_equal(oracle.bf16_bits_to_f64(y2), oracle.bf16_bits_to_f64(y) * 0.25)
    check(p, y2, alpha=0.25)


@pytest.mark.parametrize("m,N,K", [(256, 57344, 8192), (16, 8192, 28672), (256, 10240, 8192)])
def test_native_llama_shapes_sampled(m, N, K):
    p = synth.make_random(m, N, K, 1, seed=m + N, scale_lo=-6, scale_hi=2)
    _say("native sampled", m, N, K)
    y = run_native(p)
    assert np.isfinite(oracle.bf16_bits_to_f64(y)).all()
    rng = np.random.Generator(np.random.PCG64(N))
    rows = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.choice(N, 96, replace=False)]))
    check(p, y, rows)


def test_native_repeat_bit_identical():
    p = synth.make_random(256, 4096, 8192, 1, seed=21)
    _say("native determinism")
    a, b = run_native(p, reps=2)
    assert np.array_equal(a, b)


def test_native_binding_rejects_host_and_misshaped_tensors():
    # native_repack returns CPU tensors: handing them on unuploaded would give
    # the kernel host pointers, so the binding refuses them before any launch
    p = synth.make_random(16, 64, 512, 1, seed=23)
    wq, sq = F.native_repack(p.codes, p.scales, p.N, p.K)
    A = torch.from_numpy(p.a_bits.view(np.int16)).cuda().view(torch.bfloat16)
    _say("native binding checks")
    with pytest.raises(ValueError):
        F.gemm_native(A, wq, sq, p.N, p.K)
    wq_d, sq_d = wq.cuda(), sq.cuda()
    with pytest.raises(ValueError):
        F.gemm_native(A, wq_d, sq, p.N, p.K)
    with pytest.raises(ValueError):
        F.gemm_native(A, wq_d[:-16], sq_d, p.N, p.K)
    with pytest.raises(ValueError):
        F.gemm_native(A, wq_d, sq_d, p.N, p.K, out=torch.empty((16, 64), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        F.gemm_native(A, wq_d, sq_d, p.N, p.K, out=torch.empty((16, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        F.gemm_native(A, wq_d, sq_d, p.N, p.K, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    y = F.gemm_native(A, wq_d, sq_d, p.N, p.K)   # the valid call still works
    torch.cuda.synchronize()
    check(p, _bits(y))


def test_native_split_captured_in_a_graph_replays():
    # activation quantizer + FP4 GEMM + reduce of a K split, captured once and
    # replayed with new activations: every replay equals an eager call
    m, N, K = 16, 1024, 8192
    p = synth.make_random(m, N, K, 1, seed=31)
    wq, sq = F.native_repack(p.codes, p.scales, N, K)
    wq, sq = wq.cuda(), sq.cuda()
    need = F.native_workspace_size(m, N, K)
    _say("native graph replay", need)
    A = torch.from_numpy(p.a_bits.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty((m, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        F.gemm_native(A, wq, sq, N, K, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        F.gemm_native(A, wq, sq, N, K, out=out, workspace=ws)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(13)
    for rep in range(3):
        A.copy_(torch.randn((m, K), generator=gen).to(torch.bfloat16).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _bits(out)
        want = _bits(F.gemm_native(A, wq, sq, N, K))
        torch.cuda.synchronize()
        assert np.array_equal(got, want), f"replay {rep} differs from the eager call"
    a_bits = A.view(torch.int16).cpu().numpy().view(np.uint16)
    check(synth.Problem("native_graph", m, N, K, 1, a_bits, p.codes, p.scales, 31), got)


def test_native_at_its_activation_limit():
    """m = 4095 rows of K = 2^20 - 512: the quantized activations (m rounded
    to 128, Kp / 2 bytes per row) are 1 MiB short of 2^31 bytes and A is
    8.6 GB.  A's rows are drawn from 32 distinct seeded rows (the activation
    quantizer works per row), so the oracle computes 32 rows and every output
    row is held to its source row's tolerance."""
    m, N, K = 4095, 24, (1 << 20) - 512
    assert -(-m // 128) * 128 * K // 2 < (1 << 31) <= -(-m // 128) * 128 * (K + 512) // 2
    pool = synth.make_random(32, N, K, 1, seed=4095)
    src = np.random.Generator(np.random.PCG64(m)).integers(0, 32, size=m)
    _say("native at its activation limit", m, N, K)
    wq, sq = F.native_repack(pool.codes, pool.scales, N, K)
    rows = torch.from_numpy(np.ascontiguousarray(pool.a_bits).view(np.int16)).cuda().view(torch.bfloat16)
    A = rows.index_select(0, torch.from_numpy(src).cuda()).contiguous()
    y = F.gemm_native(A, wq.cuda(), sq.cuda(), N, K)
    torch.cuda.synchronize()
    del A
    y_bits = _bits(y)
    del y
    torch.cuda.empty_cache()
    y_ref, bound = oracle.native_reference(pool.a_bits, pool.codes, pool.scales, K)
    ok = oracle.check_tolerance(y_bits, y_ref[src], bound[src])
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} outputs out of tolerance"
