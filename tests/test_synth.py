"""Seeded input generators: shapes, determinism and the stated distributions."""

import numpy as np
import torch

from mixed_precision_bf16_amd import synth


def test_config_cases_cover_the_five_workloads():
    assert [c[3:6] for c in synth.config_cases(0)] == [(16, 512, 1024)]
    assert [c[4:6] for c in synth.config_cases(1)] == [(10240, 8192), (8192, 8192), (57344, 8192), (8192, 28672)]
    assert {c[3] for c in synth.config_cases(2)} == {256}
    assert len(synth.config_cases(3)) == 8 and {c[6] for c in synth.config_cases(3)} == {synth.FMT_MXFP4}
    assert sorted({c[3] for c in synth.config_cases(4)}) == [1, 7, 33, 100, 255]


def test_tiny_config_is_deterministic_and_in_domain():
    p = synth.make_problem(0, 0, 0)
    q = synth.make_problem(0, 0, 0)
    assert p.seed == 1_000_000
    assert np.array_equal(p.codes, q.codes) and np.array_equal(p.scales, q.scales)
    assert np.array_equal(p.a_bits, q.a_bits)
    assert p.codes.shape == (512, 512) and p.scales.shape == (512, 64) and p.a_bits.shape == (16, 1024)
    nib = np.concatenate([p.codes & 15, p.codes >> 4])
    assert not np.any(nib == 8), "no negative zero codes"
    assert set(np.unique(nib)) == set(range(16)) - {8}
    # E4M3 scales are positive and within [2^-4, 2^2] (bytes 0x18..0x48)
    assert p.scales.min() >= 0x18 and p.scales.max() <= 0x48
    a = torch.from_numpy(p.a_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert abs(a.mean()) < 0.05 and 0.9 < a.std() < 1.1


def test_mxfp4_scale_bytes():
    p = synth.make_random(4, 64, 256, synth.FMT_MXFP4, seed=3, scale_lo=-6, scale_hi=2)
    assert p.scales.shape == (64, 8)
    assert p.scales.min() >= 121 and p.scales.max() <= 129


def test_edge_overrides():
    p = synth.make_problem(4, 0, 1)          # N=1000, m=7, K=8192
    assert (p.m, p.N, p.K) == (7, 1000, 8192)
    seq = [0, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15, 7]
    row0 = []
    for b in p.codes[0, :8]:
        row0 += [int(b) & 15, int(b) >> 4]
    assert row0 == seq
    assert not np.any(p.codes[-1, (8192 - 16) // 2:])
    a = torch.from_numpy(p.a_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.abs(a).max() > 8.0, "outliers present"
