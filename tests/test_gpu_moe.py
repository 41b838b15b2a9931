"""GPU parity of the grouped MoE GEMM (fp4_moe_gemm, through the C ABI)
against the CPU MoE oracle (oracle.moe_reference).

Bar: every listed output row within |y - y_ref| <= 8e-3 |y_ref| + 2e-3 B
element by element (B = |w| sum_k |a_k w_k|), every listed row finite, rows
not listed untouched (they keep a NaN sentinel), repeated runs bit-identical.
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


def upload_experts(p):
    parts = [F.repack(p.codes[e], p.scales[e], p.N, p.K, p.fmt) for e in range(p.E)]
    wq = torch.from_numpy(np.concatenate([w.numpy() if hasattr(w, "numpy") else w for w, _ in parts])).cuda()
    sq = torch.from_numpy(np.concatenate([s.numpy() if hasattr(s, "numpy") else s for _, s in parts])).cuda()
    return wq, sq


def run_moe(p, reps=1):
    wq, sq = upload_experts(p)
    A = torch.from_numpy(np.ascontiguousarray(p.a_bits).view(np.int16)).cuda().view(torch.bfloat16)
    ids = torch.from_numpy(p.sorted_ids).cuda()
    off = torch.from_numpy(p.offsets).cuda()
    tw = torch.from_numpy(p.topw).cuda() if p.topw is not None else None
    outs = []
    for _ in range(reps):
        out = torch.full((p.out_rows, p.N), float("nan"), dtype=torch.bfloat16, device="cuda")
        F.moe_gemm(A, wq, sq, ids, off, p.N, p.K, p.fmt, p.E, p.a_div, p.out_rows, topk_weights=tw, out=out)
        torch.cuda.synchronize()
        outs.append(_bits(out))
    return outs if reps > 1 else outs[0]


def check(p, y_bits, cols=None):
    codes, scales = (p.codes, p.scales) if cols is None else (p.codes[:, cols], p.scales[:, cols])
    y_ref, bound, written = oracle.moe_reference(p.a_bits, codes, scales, p.sorted_ids, p.offsets, p.topw, p.a_div,
                                                 p.out_rows, p.K, p.fmt)
    yb = y_bits if cols is None else y_bits[:, cols]
    y = oracle.bf16_bits_to_f64(yb)
    assert np.isnan(y[~written]).all(), f"{p.name}: rows not listed were written"
    assert np.isfinite(oracle.bf16_bits_to_f64(y_bits[written])).all(), f"{p.name}: non-finite outputs"
    ok = oracle.check_tolerance(yb[written], y_ref[written], bound[written])
    if not ok.all():
        i, n = np.argwhere(~ok)[0]
        raise AssertionError(f"{p.name}: {int((~ok).sum())} of {ok.size} out of tolerance; first at row "
                             f"{np.flatnonzero(written)[i]}, col {n}: gpu={y[written][i, n]!r} "
                             f"ref={y_ref[written][i, n]!r} bound={bound[written][i, n]!r}")


# (T, topk, E, N, K, fmt, per_assignment_a, with_weights, skew)
CASES = [
    (5, 2, 4, 40, 64, 1, False, True, 0.0),
    (16, 4, 8, 300, 2880, 1, False, True, 0.0),
    (16, 4, 8, 300, 2880, 0, False, False, 0.0),
    (64, 4, 16, 130, 512, 1, True, True, 1.5),     # skewed: heavy experts span several 16-row blocks
    (40, 1, 2, 48, 128, 0, False, True, 0.0),       # mean 20 rows per expert: 32-row blocks
    (128, 2, 4, 64, 256, 0, True, False, 0.0),      # mean 64 rows per expert: 64-row blocks
    (7, 3, 64, 24, 96, 1, False, True, 0.0),        # most experts empty
    (33, 2, 5, 1000, 544, 0, False, True, 2.0),     # ragged N and K
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}_k{}_E{}_N{}_K{}_f{}_{}{}_s{}".format(
    *c[:6], "pa" if c[6] else "pt", "w" if c[7] else "", c[8]))
def test_moe_full_oracle(case):
    T, topk, E, N, K, fmt, pa, ww, skew = case
    p = synth.make_moe(T, topk, E, N, K, fmt, seed=1000 + T * 7 + E, per_assignment_a=pa, with_weights=ww,
                       skew=skew)
    _say("moe", p.name, "per-assignment A" if pa else "per-token A", "weights" if ww else "", skew)
    check(p, run_moe(p))


@pytest.mark.parametrize("T", [16, 256])
def test_moe_128_experts_sampled(T):
    """128 experts, top-4, N = 5760 (fused gate/up), K = 2880, MXFP4: output
    columns sampled (the first and last 16-row tiles and 64 random ones) for
    every listed row."""
    p = synth.make_moe(T, 4, 128, 5760, 2880, 1, seed=77 + T)
    _say("moe sampled", p.name)
    y = run_moe(p)
    rng = np.random.Generator(np.random.PCG64(T))
    cols = np.unique(np.concatenate([np.arange(16), np.arange(5760 - 16, 5760), rng.choice(5760, 64, replace=False)]))
    written = np.zeros(p.out_rows, bool)
    written[p.sorted_ids] = True
    assert np.isfinite(oracle.bf16_bits_to_f64(y[written])).all()
    check(p, y, cols)


def test_moe_repeat_bit_identical():
    p = synth.make_moe(32, 4, 16, 520, 1024, 0, seed=5, skew=1.0)
    _say("moe determinism")
    a, b = run_moe(p, reps=2)
    assert np.array_equal(a, b)


def test_moe_ids_out_of_range_are_skipped():
    """ids >= out_rows (or < 0) write nothing; activation rows past a_rows
    read as zero."""
    p = synth.make_moe(6, 2, 3, 32, 64, 0, seed=8)
    ids = p.sorted_ids.copy()
    ids[0] = p.out_rows + 5
    ids[-1] = -3
    q = synth.MoeProblem(p.name, p.T, p.topk, p.E, p.N, p.K, p.fmt, p.a_div, p.a_bits, p.codes, p.scales,
                         ids, p.offsets, None, p.seed)
    _say("moe out-of-range ids")
    wq, sq = upload_experts(q)
    A = torch.from_numpy(np.ascontiguousarray(q.a_bits).view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.full((q.out_rows, q.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    F.moe_gemm(A, wq, sq, torch.from_numpy(ids).cuda(), torch.from_numpy(q.offsets).cuda(), q.N, q.K, q.fmt, q.E,
               q.a_div, q.out_rows, out=out)
    torch.cuda.synchronize()
    y = oracle.bf16_bits_to_f64(_bits(out))
    keep = ids[(ids >= 0) & (ids < q.out_rows)]
    ref_ids = np.where((ids >= 0) & (ids < q.out_rows), ids, -1)
    # oracle over the valid ids only
    valid = [i for i in range(len(ids)) if 0 <= ids[i] < q.out_rows]
    vids = ids[valid]
    voff = np.array([sum(1 for i in valid if i < o) for o in q.offsets], dtype=np.int32)
    y_ref, bound, written = oracle.moe_reference(q.a_bits, q.codes, q.scales, vids, voff, None, q.a_div, q.out_rows,
                                                 q.K, q.fmt)
    assert set(np.flatnonzero(written)) == set(keep.tolist()) and ref_ids is not None
    assert np.isnan(y[~written]).all()
    assert oracle.check_tolerance(_bits(out)[written], y_ref[written], bound[written]).all()


def test_moe_grid_near_its_limit_full_oracle():
    """4096 experts (the largest E) and 960000 assignments with one activation
    row each: 960000 / 16 + 4096 = 64096 row blocks of the 65535 a launch may
    have; every listed row against the full MoE oracle."""
    p = synth.make_moe(240000, 4, 4096, 64, 256, 1, seed=4096, per_assignment_a=True)
    assert p.sorted_ids.size // 16 + p.E <= 65535
    _say("moe grid near its limit", p.name)
    check(p, run_moe(p))


def test_moe_experts_past_4_gib_sampled():
    """4096 NVFP4 experts of 2048 x 2048: 8 GiB of packed codes, so expert
    offsets pass 2^31 and 2^32 bytes.  The packed experts are seeded random
    bytes made on the device (valid scale bytes only); a sample of experts
    (the first, the last, those around the 2^31- and 2^32-byte offsets and
    random ones, each with at least one assignment) get host-drawn weights,
    and their rows are checked against the MoE oracle on those experts."""
    T, topk, E, N, K, fmt = 8192, 4, 4096, 2048, 2048, 0
    sorted_ids, offsets, topw = synth.moe_routing(T, topk, E, seed=44)
    counts = np.diff(offsets)
    nw, ns = F.repack_size(N, K, fmt)
    edges = [x for b in (1 << 31, 1 << 32) for x in (b // nw - 1, b // nw)]
    rng = np.random.Generator(np.random.PCG64(45))
    want = sorted({0, 1, E - 2, E - 1, *edges, *(int(x) for x in rng.choice(E, 20, replace=False))})
    sample = [e for e in want if counts[e] > 0]
    assert any(e * nw >= (1 << 32) for e in sample) and any((1 << 31) <= e * nw < (1 << 32) for e in sample)
    _say("moe experts past 4 GiB", T, topk, E, N, K, sample)

    gen = torch.Generator(device="cuda")
    gen.manual_seed(46)
    wq = torch.randint(0, 256, (E * nw,), dtype=torch.uint8, device="cuda", generator=gen)
    sq = torch.randint(0x18, 0x49, (E * ns,), dtype=torch.uint8, device="cuda", generator=gen)
    codes, scales = [], []
    for i, e in enumerate(sample):
        w = synth.make_random(1, N, K, fmt, seed=500 + i)
        twq, tsq = F.repack(w.codes, w.scales, N, K, fmt)
        wq[e * nw:(e + 1) * nw].copy_(torch.from_numpy(twq))
        sq[e * ns:(e + 1) * ns].copy_(torch.from_numpy(tsq))
        codes.append(w.codes)
        scales.append(w.scales)
    a_bits = synth.make_random(T, 1, K, fmt, seed=47).a_bits
    A = torch.from_numpy(np.ascontiguousarray(a_bits).view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.full((T * topk, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    F.moe_gemm(A, wq, sq, torch.from_numpy(sorted_ids).cuda(), torch.from_numpy(offsets).cuda(), N, K, fmt, E,
               topk, T * topk, topk_weights=torch.from_numpy(topw).cuda(), out=out)
    torch.cuda.synchronize()
    del wq, sq
    y_bits = _bits(out)
    del out
    torch.cuda.empty_cache()
    assert np.isfinite(oracle.bf16_bits_to_f64(y_bits)).all(), "every assignment row is written and finite"
    sub_ids = np.concatenate([sorted_ids[offsets[e]:offsets[e + 1]] for e in sample])
    sub_off = np.concatenate([[0], np.cumsum([counts[e] for e in sample])]).astype(np.int32)
    y_ref, bound, written = oracle.moe_reference(a_bits, np.stack(codes), np.stack(scales), sub_ids, sub_off, topw,
                                                 topk, T * topk, K, fmt)
    ok = oracle.check_tolerance(y_bits[written], y_ref[written], bound[written])
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} outputs of the sampled experts out of tolerance"
