"""Seeded synthetic inputs for the BF16 x FP4 GEMM.

This module only draws random bytes and BF16 activations; it holds none of the
method's arithmetic (no decoding, no dequantization, no products).  Both the
GPU path and the CPU checker receive exactly the arrays produced here.

Workloads.  The Petit blog ("Optimizing FP4 Mixed-Precision Inference on AMD
GPUs", section "Detailed performance analysis") measures the GEMM at the real
weight-matrix sizes of Llama 3 70B serving, at m = 16 (decode) and m = 256
(prefill).  No weights are available, so seeded random tensors of those shapes
stand in for them:

* codes: uniform over the 15 E2M1 codes other than negative zero (the
  petit-kernel page, "Known limitations": inputs carry no negative zeros);
* NVFP4 scales: E4M3 rounding (round to nearest even) of 2^u, u ~ U(-4, 2);
* MXFP4 scales: E8M0 byte 127 + e, e uniform over the integers -6..2;
* A: float32 N(0, 1) rounded to BF16 (nearest even), or to FP16 for the
  FP16-activation variant (``act="f16"``; same float32 draws).

The edge sweep adds 1 % outliers ~ N(0, sd 10) to A, forces row 0's first 16
codes to cover every code except negative zero (including +-6 and 0) and forces
the tail group of the last row to all-zero codes.

Seeds: numpy PCG64 with seed 1_000_000*(config+1) + 1000*shape_idx + m_idx;
draw order codes -> scales -> A -> overrides.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

FMT_NVFP4 = 0
FMT_MXFP4 = 1
GROUP = {FMT_NVFP4: 16, FMT_MXFP4: 32}

# Llama 3 70B linear-layer weight shapes (N, K): fused QKV, attention output,
# fused gate/up projection, down projection.
LLAMA3_70B_LAYERS = (
    ("qkv", 10240, 8192),
    ("o", 8192, 8192),
    ("gate_up", 57344, 8192),
    ("down", 8192, 28672),
)


@dataclass
class Problem:
    """One GEMM instance: A [m][K] BF16 (or FP16) bits, codes [N][K/2], scales [N][K/G]."""
    name: str
    m: int
    N: int
    K: int
    fmt: int
    a_bits: np.ndarray
    codes: np.ndarray
    scales: np.ndarray
    seed: int
    act: str = "bf16"

    @property
    def group(self) -> int:
        return GROUP[self.fmt]


def config_cases(config: int):
    """List of (name, shape_idx, m_idx, m, N, K, fmt) for one workload config."""
    cases = []
    if config == 0:
        cases.append(("tiny", 0, 0, 16, 512, 1024, FMT_NVFP4))
    elif config in (1, 2):
        m = 16 if config == 1 else 256
        for si, (nm, N, K) in enumerate(LLAMA3_70B_LAYERS):
            cases.append((f"{nm}_m{m}", si, 0, m, N, K, FMT_NVFP4))
    elif config == 3:
        for si, (nm, N, K) in enumerate((("down", 8192, 28672), ("gate_up", 57344, 8192))):
            for mi, m in enumerate((1, 4, 8, 16)):
                cases.append((f"mx_{nm}_m{m}", si, mi, m, N, K, FMT_MXFP4))
    elif config == 4:
        for si, N in enumerate((1000, 8200)):
            for mi, m in enumerate((1, 7, 33, 100, 255)):
                cases.append((f"edge_N{N}_m{m}", si, mi, m, N, 8192, FMT_NVFP4))
    else:
        raise ValueError(f"unknown config {config}")
    return cases


def _draw_codes(rng, N, K):
    """Packed codes [N][K/2]: element 2j in the low nibble, 2j+1 in the high."""
    x = rng.integers(0, 15, size=(N, K), dtype=np.uint8)
    x += (x >= 8).astype(np.uint8)          # skip 8 (negative zero)
    return (x[:, 0::2] | (x[:, 1::2] << 4)).astype(np.uint8)


def _e4m3_bytes_of(values_f32: np.ndarray) -> np.ndarray:
    """Round float32 values to E4M3 with the library cast (nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _bf16_bits_of(values_f32: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 with the library cast (nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _f16_bits_of(values_f32: np.ndarray) -> np.ndarray:
    """Round float32 values to FP16 with the library cast (nearest even)."""
    return np.ascontiguousarray(values_f32, dtype=np.float32).astype(np.float16).view(np.uint16).copy()


def _act_bits_of(values_f32: np.ndarray, act: str) -> np.ndarray:
    if act == "bf16":
        return _bf16_bits_of(values_f32)
    if act == "f16":
        return _f16_bits_of(values_f32)
    raise ValueError(f"unknown activation type {act}")


def _draw_scales(rng, N, K, fmt):
    G = GROUP[fmt]
    if fmt == FMT_NVFP4:
        u = rng.uniform(-4.0, 2.0, size=(N, K // G))
        return _e4m3_bytes_of(np.exp2(u).astype(np.float32))
    e = rng.integers(-6, 3, size=(N, K // G))
    return (127 + e).astype(np.uint8)


def _draw_a(rng, m, K, act="bf16"):
    return _act_bits_of(rng.standard_normal(size=(m, K), dtype=np.float32), act)


def make_problem(config: int, shape_idx: int, m_idx: int, act: str = "bf16") -> Problem:
    """Build the seeded inputs of one case of one workload config."""
    for (name, si, mi, m, N, K, fmt) in config_cases(config):
        if si == shape_idx and mi == m_idx:
            break
    else:
        raise ValueError(f"no case ({shape_idx}, {m_idx}) in config {config}")
    seed = 1_000_000 * (config + 1) + 1000 * shape_idx + m_idx
    rng = np.random.Generator(np.random.PCG64(seed))
    codes = _draw_codes(rng, N, K)
    scales = _draw_scales(rng, N, K, fmt)
    a_bits = _draw_a(rng, m, K, act)
    if config == 4:
        _edge_overrides(rng, a_bits, codes, m, N, K, act)
    return Problem(name, m, N, K, fmt, a_bits, codes, scales, seed, act)


def _edge_overrides(rng, a_bits, codes, m, N, K, act="bf16"):
    # 1 % of A replaced by N(0, sd 10) outliers.
    mask = rng.random(size=(m, K)) < 0.01
    out = rng.standard_normal(size=(m, K), dtype=np.float32) * np.float32(10.0)
    a_bits[mask] = _act_bits_of(out, act)[mask]
    # Row 0, k = 0..15: every code except negative zero, then code 7 (+6).
    seq = np.array([0, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15, 7], dtype=np.uint8)
    codes[0, 0:8] = seq[0::2] | (seq[1::2] << 4)
    # Tail group (16 elements) of the last row: all-zero codes.
    codes[N - 1, (K - 16) // 2:] = 0


def make_random(m: int, N: int, K: int, fmt: int, seed: int, *,
                scale_lo: float = -4.0, scale_hi: float = 2.0,
                allow_neg_zero: bool = False, a_scale: float = 1.0, act: str = "bf16") -> Problem:
    """Free-shape case with the same distributions (for ragged/edge tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    G = GROUP[fmt]
    if allow_neg_zero:
        x = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        codes = (x[:, 0::2] | (x[:, 1::2] << 4)).astype(np.uint8)
    else:
        codes = _draw_codes(rng, N, K)
    if fmt == FMT_NVFP4:
        u = rng.uniform(scale_lo, scale_hi, size=(N, K // G))
        scales = _e4m3_bytes_of(np.exp2(u).astype(np.float32))
    else:
        e = rng.integers(int(scale_lo), int(scale_hi) + 1, size=(N, K // G))
        scales = (127 + e).astype(np.uint8)
    a = rng.standard_normal(size=(m, K), dtype=np.float32) * np.float32(a_scale)
    a_bits = _act_bits_of(a, act)
    return Problem(f"rand_m{m}_N{N}_K{K}_f{fmt}_{act}", m, N, K, fmt, a_bits, codes, scales, seed, act)


@dataclass
class MoeProblem:
    """Grouped MoE instance: A [a_rows][K] BF16 bits, expert codes [E][N][K/2]
    and scales [E][N][K/G], assignment ids grouped by expert (sorted_ids,
    offsets [E+1]), routing weights per assignment id (or None)."""
    name: str
    T: int
    topk: int
    E: int
    N: int
    K: int
    fmt: int
    a_div: int
    a_bits: np.ndarray
    codes: np.ndarray
    scales: np.ndarray
    sorted_ids: np.ndarray
    offsets: np.ndarray
    topw: np.ndarray | None
    seed: int

    @property
    def out_rows(self) -> int:
        return self.T * self.topk

    @property
    def a_rows(self) -> int:
        return self.a_bits.shape[0]


def _moe_routing(rng, T, topk, E, with_weights, skew):
    if skew > 0:
        p = (np.arange(E) + 1.0) ** -skew
        p = p[np.argsort(rng.permutation(E))] / p.sum()
    else:
        p = None
    route = np.stack([rng.choice(E, size=topk, replace=False, p=p) for _ in range(T)])   # [T][topk]
    topw = rng.random(size=T * topk).astype(np.float32) if with_weights else None
    ids = np.arange(T * topk, dtype=np.int64)
    expert_of = route.reshape(-1)
    order = np.argsort(expert_of, kind="stable")
    sorted_ids = ids[order].astype(np.int32)
    counts = np.bincount(expert_of, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return sorted_ids, offsets, topw


def moe_routing(T: int, topk: int, E: int, seed: int, *, with_weights: bool = True, skew: float = 0.0):
    """The routing part of make_moe alone (same seed, same draws): returns
    (sorted_ids, offsets, topw)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _moe_routing(rng, T, topk, E, with_weights, skew)


def make_moe(T: int, topk: int, E: int, N: int, K: int, fmt: int, seed: int, *, per_assignment_a: bool = False,
             with_weights: bool = True, skew: float = 0.0) -> MoeProblem:
    """Seeded synthetic MoE routing and weights.  Each token picks topk
    distinct experts, uniformly (skew = 0) or with probability proportional
    to (rank + 1)^-skew over a random expert order (skew > 0 makes a few
    experts hold many rows and leaves others empty); assignment id =
    token * topk + slot.  Routing weights are uniform in [0, 1) rounded to
    FP32.  A holds one row per token (a_div = topk) or, with
    per_assignment_a, one row per assignment (a_div = 1).  Codes, scales and
    activations follow the dense generators' distributions.  Draw order:
    routing -> weights -> codes -> scales -> A."""
    rng = np.random.Generator(np.random.PCG64(seed))
    sorted_ids, offsets, topw = _moe_routing(rng, T, topk, E, with_weights, skew)
    codes = np.stack([_draw_codes(rng, N, K) for _ in range(E)])
    scales = np.stack([_draw_scales(rng, N, K, fmt) for _ in range(E)])
    a_rows = T * topk if per_assignment_a else T
    a_bits = _draw_a(rng, a_rows, K)
    return MoeProblem(f"moe_T{T}_k{topk}_E{E}_N{N}_K{K}_f{fmt}", T, topk, E, N, K, fmt,
                      1 if per_assignment_a else topk, a_bits, codes, scales, sorted_ids, offsets, topw, seed)

