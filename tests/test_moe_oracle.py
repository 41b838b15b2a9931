"""Pins of the MoE oracle (oracle.moe_reference) against facts outside it.

* The single-expert identity routing is the dense GEMM, whose oracle is pinned
  in test_oracle.py: the two must agree exactly.
* Exact rational brute force of a tiny routed problem (tokens routed to two
  experts each, one expert left empty, routing weights that are exact binary
  fractions), written with plain loops over the definition.
* The order of the ids inside an expert's range does not matter.
Planted mistakes (wrong expert, routing weight dropped, activation row taken
as the assignment id) each fail a pin.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp4_oracle as O
from oracle import moe_oracle as MO

pytestmark = pytest.mark.filterwarnings("ignore")


def _a_bits(rows):
    return torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _e2m1(code):
    pos = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
           Fraction(6)]
    v = pos[code & 7]
    return -v if code & 8 else v


def _scale(byte, fmt):
    t = torch.tensor([byte], dtype=torch.uint8)
    dt = torch.float8_e4m3fn if fmt == 0 else torch.float8_e8m0fnu
    return Fraction(float(t.view(dt).to(torch.float64)[0]))


def _routed_problem(seed=3, fmt=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    T, topk, E, N, K = 3, 2, 4, 2, 64
    G = 16 if fmt == 0 else 32
    a = rng.integers(-4, 5, size=(T, K)).astype(np.float32) / 2          # exact in BF16
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    scales = (rng.integers(0x30, 0x40, size=(E, N, K // G)) if fmt == 0
              else rng.integers(124, 130, size=(E, N, K // G))).astype(np.uint8)
    # token t -> experts route[t]; expert 3 gets nothing
    route = [[2, 0], [0, 1], [1, 2]]
    ids = [[] for _ in range(E)]
    for t in range(T):
        for j, e in enumerate(route[t]):
            ids[e].append(t * topk + j)
    sorted_ids = np.array([i for e in range(E) for i in ids[e]], dtype=np.int32)
    offsets = np.cumsum([0] + [len(x) for x in ids]).astype(np.int32)
    topw = np.array([0.75, 0.25, 0.5, 0.5, 1.0, 0.125], dtype=np.float32)
    return dict(a=a, codes=codes, scales=scales, route=route, sorted_ids=sorted_ids, offsets=offsets, topw=topw,
                T=T, topk=topk, E=E, N=N, K=K, fmt=fmt, G=G)


def pin_dense_special_case(mo):
    rng = np.random.Generator(np.random.PCG64(5))
    m, N, K = 5, 7, 64
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x48, size=(N, K // 16)).astype(np.uint8)
    a_bits = _a_bits(rng.standard_normal((m, K)).astype(np.float32).tolist())
    y, b = O.gemm_reference(a_bits, codes, scales, K, 0)
    ym, bm, wr = mo.moe_reference(a_bits, codes[None], scales[None], np.arange(m), np.array([0, m]), None, 1, m,
                                  K, 0)
    assert wr.all()
    assert np.array_equal(y, ym) and np.array_equal(b, bm)


def pin_bruteforce(mo):
    for fmt in (0, 1):
        p = _routed_problem(fmt=fmt)
        out_rows = p["T"] * p["topk"]
        y, b, wr = mo.moe_reference(_a_bits(p["a"].tolist()), p["codes"], p["scales"], p["sorted_ids"],
                                    p["offsets"], p["topw"], p["topk"], out_rows, p["K"], fmt)
        assert wr.all()
        for t in range(p["T"]):
            for j, e in enumerate(p["route"][t]):
                aid = t * p["topk"] + j
                w = Fraction(float(p["topw"][aid]))
                for n in range(p["N"]):
                    s = Fraction(0)
                    babs = Fraction(0)
                    for k in range(p["K"]):
                        byte = int(p["codes"][e, n, k // 2])
                        code = byte & 15 if k % 2 == 0 else byte >> 4
                        term = Fraction(float(p["a"][t, k])) * _e2m1(code) * _scale(int(p["scales"][e, n, k // p["G"]]),
                                                                                      fmt)
                        s += term
                        babs += abs(term)
                    assert Fraction(float(y[aid, n])) == w * s, (fmt, t, j, n)
                    assert Fraction(float(b[aid, n])) == abs(w) * babs


def pin_order_invariance(mo):
    p = _routed_problem(seed=9)
    out_rows = p["T"] * p["topk"]
    args = (_a_bits(p["a"].tolist()), p["codes"], p["scales"])
    y0, _, _ = mo.moe_reference(*args, p["sorted_ids"], p["offsets"], p["topw"], p["topk"], out_rows, p["K"], 0)
    ids = p["sorted_ids"].copy()
    for e in range(p["E"]):
        ids[p["offsets"][e]:p["offsets"][e + 1]] = ids[p["offsets"][e]:p["offsets"][e + 1]][::-1]
    y1, _, _ = mo.moe_reference(*args, ids, p["offsets"], p["topw"], p["topk"], out_rows, p["K"], 0)
    assert np.array_equal(y0, y1)


ALL_PINS = [pin_dense_special_case, pin_bruteforce, pin_order_invariance]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_moe_oracle_pin(pin):
    pin(MO)


def test_duplicate_ids_rejected():
    p = _routed_problem()
    ids = p["sorted_ids"].copy()
    ids[1] = ids[0]
    with pytest.raises(ValueError):
        MO.moe_reference(_a_bits(p["a"].tolist()), p["codes"], p["scales"], ids, p["offsets"], None, 2, 6, p["K"], 0)


class _Mutant:
    def __init__(self, fn):
        self.moe_reference = fn


def _mut_expert_shift(a_bits, codes, scales, ids, off, topw, a_div, out_rows, K, fmt, act="bf16"):
    return MO.moe_reference(a_bits, np.roll(codes, 1, axis=0), np.roll(scales, 1, axis=0), ids, off, topw, a_div,
                            out_rows, K, fmt, act)


def _mut_no_weight(a_bits, codes, scales, ids, off, topw, a_div, out_rows, K, fmt, act="bf16"):
    return MO.moe_reference(a_bits, codes, scales, ids, off, None, a_div, out_rows, K, fmt, act)


def _mut_row_is_id(a_bits, codes, scales, ids, off, topw, a_div, out_rows, K, fmt, act="bf16"):
    bits = np.asarray(a_bits)
    rows = max(out_rows, bits.shape[0])
    big = np.zeros((rows, bits.shape[1]), dtype=bits.dtype)
    big[:bits.shape[0]] = bits
    return MO.moe_reference(big, codes, scales, ids, off, topw, 1, out_rows, K, fmt, act)


@pytest.mark.parametrize("name,fn", [("expert index shifted", _mut_expert_shift),
                                     ("routing weight dropped", _mut_no_weight),
                                     ("activation row = assignment id", _mut_row_is_id)])
def test_planted_mistake_is_caught(name, fn):
    failures = 0
    for pin in ALL_PINS:
        try:
            pin(_Mutant(fn))
        except AssertionError:
            failures += 1
    assert failures, f"planted mistake '{name}' passed every pin"
