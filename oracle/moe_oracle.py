"""Plain float64 oracle of the grouped ("fused") mixture-of-experts GEMM.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
uses this module.

What is computed, and where the pages say so
--------------------------------------------
The petit-kernel PyPI page ("Features") lists fused MoE kernels for BF16
activations and MXFP4 weights beside the dense GEMM, and says no more about
them.  Read here in the plainest way that the dense GEMM supports: every
expert e has its own FP4 weight matrix W_e [N][K] (same formats and dequant as
the dense GEMM); each (token, expert) assignment has an id, and the ids routed
to expert e are listed in sorted_ids[offsets[e] : offsets[e + 1]]; the output
row of assignment id is

    y[id] = w[id] * ( A[id // a_div] . dequant(W_e)^T )

where a_div maps an assignment to its activation row (the number of experts
per token when A holds one row per token, 1 when A already holds one row per
assignment) and w is an optional per-assignment routing weight (1 when
absent).  Rows whose id is not listed are not part of the result.
"""

from __future__ import annotations

import numpy as np

from .fp4_oracle import act_bits_to_f64, dequant_weights


def moe_reference(a_bits, codes, scales, sorted_ids, offsets, topw, a_div: int, out_rows: int, K: int, fmt: int,
                  act: str = "bf16"):
    """Returns (y_ref [out_rows][N], bound [out_rows][N], written [out_rows]).

    codes: uint8 [E][N][K/2]; scales: uint8 [E][N][K/G]; sorted_ids: int
    [P]; offsets: int [E + 1]; topw: float [out_rows] or None.  The bound is
    |w[id]| * sum_k |a_k w_k| (the dense GEMM's bound scaled by the routing
    weight).  Each id must appear at most once.
    """
    E, N = codes.shape[0], codes.shape[1]
    a = act_bits_to_f64(a_bits, act)
    ids = np.asarray(sorted_ids, dtype=np.int64)
    off = np.asarray(offsets, dtype=np.int64)
    y = np.zeros((out_rows, N))
    b = np.zeros((out_rows, N))
    written = np.zeros(out_rows, dtype=bool)
    for e in range(E):
        rows = ids[off[e]:off[e + 1]]
        if rows.size == 0:
            continue
        if written[rows].any() or np.unique(rows).size != rows.size:
            raise ValueError("assignment ids must be unique")
        w = dequant_weights(codes[e], scales[e], K, fmt)
        x = a[rows // a_div]
        s = np.ones(rows.size) if topw is None else np.asarray(topw, dtype=np.float64)[rows]
        y[rows] = s[:, None] * (x @ w.T)
        b[rows] = np.abs(s)[:, None] * (np.abs(x) @ np.abs(w).T)
        written[rows] = True
    return y, b, written
