"""Host-side tests of the C ABI: symbols, offline repack/unpack, argument checks.

No GPU is needed: repack/unpack are pure host functions and every argument
check of the device entry points runs before any HIP call.
"""

import ctypes

import numpy as np
import pytest

from mixed_precision_bf16_amd import fp4gemm as F
from mixed_precision_bf16_amd import synth


def test_library_exports_every_header_function():
    lib = F.lib()
    names = F.header_functions()
    assert set(names) == set(F._SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(8):
        assert F.lib().fp4_status_string(s)
    assert F.lib().fp4_status_string(99) == b"unknown status"


@pytest.mark.parametrize("N,K,fmt", [(1, 16, 0), (16, 512, 0), (17, 528, 0), (2, 32, 1), (33, 1056, 1),
                                     (512, 1024, 0), (100, 8192, 1)])
def test_repack_size(N, K, fmt):
    G = 16 if fmt == 0 else 32
    Np = -(-N // 16) * 16
    Kp = -(-K // 512) * 512
    assert F.repack_size(N, K, fmt) == (Np * Kp // 2, Np * Kp // G)


def _rand_weights(N, K, fmt, seed, all_codes=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    G = 16 if fmt == 0 else 32
    codes = rng.integers(0, 256 if all_codes else 1, size=(N, K // 2), dtype=np.uint8)
    hi = 0x7F if fmt == 0 else 0xFF
    scales = rng.integers(0, hi, size=(N, K // G), dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("N,K,fmt", [(1, 16, 0), (2, 32, 1), (15, 48, 0), (16, 512, 0), (17, 528, 0),
                                     (40, 1040, 0), (33, 1056, 1), (130, 2080, 1), (64, 8192, 0)])
def test_repack_roundtrip_and_padding(N, K, fmt):
    codes, scales = _rand_weights(N, K, fmt, seed=N * 1000 + K + fmt)
    wq, sq = F.repack(codes, scales, N, K, fmt)
    c2, s2 = F.unpack(wq, sq, N, K, fmt)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # the packed arrays hold the same multiset of nibbles / scale bytes plus zero padding
    nib = lambda x: np.bincount(np.concatenate([x.ravel() & 15, x.ravel() >> 4]), minlength=16)
    pad_nibbles = 2 * wq.size - 2 * codes.size
    want = nib(codes)
    want[0] += pad_nibbles
    assert np.array_equal(nib(wq), want)
    sb = np.bincount(scales.ravel(), minlength=256)
    sb[0] += sq.size - scales.size
    assert np.array_equal(np.bincount(sq, minlength=256), sb)


def test_repack_is_a_permutation_of_source_dwords():
    # Every source dword (8 consecutive k of one row) lands intact in one
    # 4-byte-aligned slot of the packed codes.
    N, K = 20, 1024
    codes = ((np.arange(N * K // 2) * 2654435761) >> 7).astype(np.uint8).reshape(N, K // 2)
    scales = np.full((N, K // 16), 0x38, np.uint8)
    wq, _ = F.repack(codes, scales, N, K, 0)
    slots = {bytes(wq[i:i + 4]) for i in range(0, wq.size, 4)}
    for n in range(N):
        for k in range(0, K, 8):
            assert bytes(codes[n, k // 2:k // 2 + 4]) in slots


def _packed_code_offset(n, k, K):
    """Documented packed-code layout: 1 KiB block per (16-row tile, 128-K chunk);
    lane 16 j + r holds 16 bytes; its dword i covers k = 128 b + 32 i + 8 j .. +7."""
    KB = -(-K // 512) * 4
    t, r = divmod(n, 16)
    b, kk = divmod(k, 128)
    i, j = kk // 32, (kk % 32) // 8
    return ((t * KB + b) * 64 + 16 * j + r) * 16 + 4 * i + (k % 8) // 2


def _packed_scale_offset(n, k, K, fmt):
    SB = -(-K // 512)
    t, r = divmod(n, 16)
    sb, c, i = k // 512, (k % 512) // 128, (k % 128) // 32
    if fmt == 0:
        return (t * SB + sb) * 512 + ((k % 32) // 16) * 256 + r * 16 + 4 * c + i
    return (t * SB + sb) * 256 + r * 16 + 4 * c + i


@pytest.mark.parametrize("N,K,fmt", [(19, 1040, 0), (33, 1056, 1)])
def test_repack_matches_documented_layout(N, K, fmt):
    codes, scales = _rand_weights(N, K, fmt, seed=77)
    G = 16 if fmt == 0 else 32
    wq, sq = F.repack(codes, scales, N, K, fmt)
    for n in range(N):
        for k in range(0, K, 2):
            assert wq[_packed_code_offset(n, k, K)] == codes[n, k // 2]
        for g in range(K // G):
            assert sq[_packed_scale_offset(n, g * G, K, fmt)] == scales[n, g]


def test_repack_synthetic_config_roundtrip():
    p = synth.make_problem(0, 0, 0)
    wq, sq = F.repack(p.codes, p.scales, p.N, p.K, p.fmt)
    c2, s2 = F.unpack(wq, sq, p.N, p.K, p.fmt)
    assert np.array_equal(c2, p.codes) and np.array_equal(s2, p.scales)


@pytest.mark.parametrize("fmt,bad", [(0, 0x80), (0, 0xB8), (0, 0x7F), (0, 0xFF), (1, 0xFF)])
def test_repack_rejects_negative_or_nan_scales(fmt, bad):
    N, K = 4, 64
    G = 16 if fmt == 0 else 32
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.full((N, K // G), 0x38 if fmt == 0 else 127, np.uint8)
    scales[2, 1] = bad
    nw, ns = F.repack_size(N, K, fmt)
    wq = np.full(nw, 0xAB, np.uint8)
    sq = np.full(ns, 0xAB, np.uint8)
    st = F.lib().fp4_repack(F._np_ptr(codes), F._np_ptr(scales), N, K, fmt, F._np_ptr(wq), F._np_ptr(sq))
    assert st == 4
    assert np.all(wq == 0xAB) and np.all(sq == 0xAB), "nothing written on error"


def test_repack_accepts_zero_scale_and_negative_zero_codes():
    N, K = 3, 32
    codes = np.full((N, K // 2), 0x88, np.uint8)
    scales = np.zeros((N, 2), np.uint8)
    wq, sq = F.repack(codes, scales, N, K, 0)
    c2, s2 = F.unpack(wq, sq, N, K, 0)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


@pytest.mark.parametrize("N,K,fmt,status", [(0, 16, 0, 2), (4, 8, 0, 2), (4, 24, 0, 2), (4, 16, 1, 2),
                                            (4, 48, 1, 2), (4, 32, 2, 3), (4, 32, -1, 3), (4, 1 << 21, 0, 2)])
def test_shape_and_format_errors(N, K, fmt, status):
    sz = ctypes.c_size_t()
    assert F.lib().fp4_repack_size(N, K, fmt, ctypes.byref(sz), ctypes.byref(sz)) == status
    assert F.lib().fp4_gemm_workspace_size(16, N, K, fmt, ctypes.byref(sz)) == status
    dummy = ctypes.c_void_p(1)
    for gemm in (F.lib().fp4_gemm, F.lib().fp4_gemm_f16):
        assert gemm(dummy, dummy, dummy, dummy, 16, N, K, fmt, None, 0, None) == status
    for deq in (F.lib().fp4_dequant, F.lib().fp4_dequant_f16):
        assert deq(dummy, dummy, dummy, N, K, fmt, None) == status


def test_gemm_argument_errors_before_any_hip_call():
    lib = F.lib()
    d = ctypes.c_void_p(1)
    z = ctypes.c_void_p(0)
    # null pointers
    for args in ((z, d, d, d), (d, z, d, d), (d, d, z, d), (d, d, d, z)):
        assert lib.fp4_gemm(*args, 16, 64, 64, 0, None, 0, None) == 1
    # negative / huge m
    assert lib.fp4_gemm(d, d, d, d, -1, 64, 64, 0, None, 0, None) == 2
    assert lib.fp4_gemm(d, d, d, d, (1 << 20) + 1, 64, 64, 0, None, 0, None) == 2
    # m = 0 is a no-op, even with null pointers
    assert lib.fp4_gemm(z, z, z, z, 0, 64, 64, 0, None, 0, None) == 0
    assert lib.fp4_gemm_f16(z, z, z, z, 0, 64, 64, 0, None, 0, None) == 0
    for args in ((z, d, d, d), (d, d, d, z)):
        assert lib.fp4_gemm_f16(*args, 16, 64, 64, 0, None, 0, None) == 1
    assert lib.fp4_dequant_f16(d, z, d, 4, 32, 0, None) == 1
    # A bytes beyond the 32-bit buffer range
    assert lib.fp4_gemm(d, d, d, d, 1 << 20, 64, 1024, 0, None, 0, None) == 2
    # repack / unpack / dequant null pointers
    assert lib.fp4_repack(z, d, 4, 32, 0, d, d) == 1
    assert lib.fp4_unpack(d, d, 4, 32, 0, z, d) == 1
    assert lib.fp4_dequant(d, z, d, 4, 32, 0, None) == 1
    sz = ctypes.c_size_t(123)
    assert lib.fp4_gemm_workspace_size(16, 64, 64, 0, None) == 1
    assert lib.fp4_gemm_workspace_size(16, 64, 64, 0, ctypes.byref(sz)) == 0


def test_moe_argument_errors_before_any_hip_call():
    lib = F.lib()
    d = ctypes.c_void_p(16)
    z = ctypes.c_void_p(0)

    def moe(A=d, wq=d, sq=d, ids=d, off=d, tw=z, C=d, a_rows=16, a_div=4, out_rows=64, P=64, E=8, N=64, K=64,
            fmt=0):
        return lib.fp4_moe_gemm(A, wq, sq, ids, off, tw, C, a_rows, a_div, out_rows, P, E, N, K, fmt, None)
    assert moe(fmt=7) == 3
    assert moe(K=24) == 2
    assert moe(E=0) == 2 and moe(E=5000) == 2
    assert moe(a_div=0) == 2 and moe(a_rows=0) == 2 and moe(out_rows=0) == 2
    assert moe(P=-1) == 2 and moe(P=(1 << 24) + 1) == 2
    # P = 0 is a no-op, even with null pointers
    assert moe(A=z, wq=z, sq=z, ids=z, off=z, C=z, P=0) == 0
    for k in ("A", "wq", "sq", "ids", "off", "C"):
        assert moe(**{k: z}) == 1, k
    # misaligned pointers
    assert moe(A=ctypes.c_void_p(8)) == 2
    assert moe(ids=ctypes.c_void_p(18)) == 2
    assert moe(tw=ctypes.c_void_p(2)) == 2
    # more row blocks than one grid column holds
    assert moe(P=1 << 24, E=4096, out_rows=1 << 24) == 2
    # A bytes beyond the 32-bit buffer range
    assert moe(a_rows=1 << 20, K=1024) == 2


def test_gemm_ex_and_quantize_argument_errors_before_any_hip_call():
    lib = F.lib()
    d = ctypes.c_void_p(16)
    z = ctypes.c_void_p(0)
    ex = lib.fp4_gemm_ex
    assert ex(d, d, d, d, 16, 64, 64, 0, 2, 1.0, None, 0, None) == 3          # act_type
    for bad in (float("nan"), float("inf"), 0.0, 2.0 ** -101, 2.0 ** 101):
        assert ex(d, d, d, d, 16, 64, 64, 0, 0, bad, None, 0, None) == 4, bad
    assert ex(z, d, d, d, 16, 64, 64, 0, 0, 0.5, None, 0, None) == 1
    assert ex(z, z, z, z, 0, 64, 64, 0, 1, 0.5, None, 0, None) == 0           # m = 0 no-op
    q = lib.fp4_quantize
    assert q(d, d, d, 4, 64, 9, 1.0, None) == 3
    assert q(d, d, d, 4, 24, 0, 1.0, None) == 2 and q(d, d, d, 4, 48, 1, 1.0, None) == 2
    assert q(d, d, d, 0, 64, 0, 1.0, None) == 2
    assert q(z, d, d, 4, 64, 0, 1.0, None) == 1 and q(d, d, z, 4, 64, 0, 1.0, None) == 1
    assert q(ctypes.c_void_p(8), d, d, 4, 64, 0, 1.0, None) == 2
    assert q(d, ctypes.c_void_p(20), d, 4, 64, 1, 1.0, None) == 2              # MXFP4 codes: 16-byte stores
    for bad in (float("nan"), -1.0, 0.0, float("inf")):
        assert q(d, d, d, 4, 64, 0, bad, None) == 4, bad


def test_native_repack_roundtrip_and_layout():
    rng = np.random.Generator(np.random.PCG64(12))
    for N, K in ((5, 64), (37, 2880), (16, 512), (130, 1056)):
        codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        scales = rng.integers(0, 255, size=(N, K // 32), dtype=np.uint8)
        wq, sq = F.native_repack(codes, scales, N, K)
        nw, ns = F.repack_size(N, K, F.MXFP4)
        assert wq.numel() == nw and sq.numel() == ns
        c2, s2 = F.native_unpack(wq, sq, N, K)
        assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
        wqn, sqn = wq.numpy(), sq.numpy()
        KB, QB = -(-K // 512) * 4, -(-K // 512)
        for _ in range(20):                      # documented offsets
            n, kb = int(rng.integers(N)), int(rng.integers(K // 32))
            t, r, c, j = n // 16, n % 16, kb // 4, kb % 4
            off = (t * KB + c) * 1024 + (16 * j + r) * 16
            assert bytes(wqn[off:off + 16]) == bytes(codes[n, kb * 16:kb * 16 + 16])
            q, s_ = kb // 16, (kb % 16) // 4
            assert sqn[(t * QB + q) * 256 + (16 * j + r) * 4 + s_] == scales[n, kb]
    lib = F.lib()
    d = ctypes.c_void_p(16)
    z = ctypes.c_void_p(0)
    assert lib.fp4_native_repack(z, d, 4, 64, d, d) == 1
    assert lib.fp4_native_repack(d, d, 4, 48, d, d) == 2                     # K % 32
    bad = np.full((2, 2), 0xFF, np.uint8)
    buf = np.zeros(4096, np.uint8)
    assert lib.fp4_native_repack(np.zeros((2, 32), np.uint8).ctypes.data_as(ctypes.c_void_p),
                                 bad.ctypes.data_as(ctypes.c_void_p), 2, 64, buf.ctypes.data_as(ctypes.c_void_p),
                                 buf.ctypes.data_as(ctypes.c_void_p)) == 4
    g = lib.fp4_gemm_native
    assert g(d, d, d, d, 16, 64, 48, 1.0, d, 1 << 20, None) == 2
    assert g(d, d, d, d, 16, 64, 64, float("nan"), d, 1 << 20, None) == 4
    assert g(z, z, z, z, 0, 64, 64, 1.0, None, 0, None) == 0
    assert g(z, d, d, d, 16, 64, 64, 1.0, d, 1 << 20, None) == 1
    assert g(d, d, d, d, 16, 64, 64, 1.0, ctypes.c_void_p(272), 1 << 20, None) == 5      # workspace alignment
    assert g(d, d, d, d, 16, 64, 64, 1.0, d, 16, None) == 5                            # workspace size
    sz = ctypes.c_size_t(0)
    assert lib.fp4_gemm_native_workspace_size(256, 57344, 8192, ctypes.byref(sz)) == 0
    assert sz.value >= 256 * 8192 // 2 + 256 * 8192 // 32


def test_python_binding_validation():
    codes, scales = _rand_weights(4, 64, 0, 1)
    with pytest.raises(ValueError):
        F.repack(codes[:, :8], scales, 4, 64, 0)
    with pytest.raises(F.Fp4Error) as e:
        F.repack_size(4, 24, 0)
    assert e.value.status == 2


def test_workspace_size_is_a_split_k_partial_buffer():
    # 0 (no K split) or S * m * N * 4 bytes with 2 <= S <= 16 and S <= K / 512,
    # a pure function of the arguments; for m <= 64 the S planes are followed
    # (at a 256-byte aligned offset) by one 8-byte arrival word per group of
    # n-tiles.
    for m, N, K, fmt in ((16, 8192, 8192, 0), (16, 57344, 8192, 0), (16, 8192, 28672, 0), (1, 8192, 28672, 1),
                         (33, 100, 544, 1), (64, 10240, 8192, 0), (7, 1000, 8192, 0), (256, 8192, 8192, 0),
                         (300, 96, 640, 0)):
        b = F.workspace_size(m, N, K, fmt)
        assert b == F.workspace_size(m, N, K, fmt)
        if b:
            S, rem = divmod(b, 4 * m * N)
            assert 2 <= S <= min(16, -(-K // 512)), (m, N, K, b)
            if m > 64 or rem == 0:  # prefill K split (also 33 <= m <= 64 on some narrower layers)
                assert rem == 0 and m > 32, (m, N, K, b)
            else:
                words = -(-N // 16)  # at most one group per 16-row n-tile
                assert 8 <= rem <= 252 + 8 * words and (b - 8 * (rem // 8)) % 4 == 0, (m, N, K, b)
    assert F.workspace_size(0, 8192, 8192, 0) == 0
    # prefill m: the split that fills the 256 CUs in the fewest rounds per unit of work
    for (m, N, K), S in (((256, 8192, 8192), 4), ((256, 10240, 8192), 3), ((256, 8192, 28672), 4),
                         ((65, 1000, 8192), 8)):
        b = F.workspace_size(m, N, K, 0)
        assert b == S * 4 * m * N, (m, N, K, b)
    assert F.workspace_size(256, 57344, 8192, 0) == 0
    assert F.new_workspace(1000, 57344, 8192, 0) is None
    # 33 <= m <= 64 on a layer of >= 128 groups of 256 columns: whole-K prefill
    # tiles, no workspace
    for m in (33, 48, 64):
        assert F.workspace_size(m, 57344, 8192, 0) == 0
        assert F.workspace_size(m, 32768, 544, 1) == 0
    # on narrower layers: the decode kernel while its grid fills the GPU and K
    # is at most 16384 (O-shaped: decode planes plus arrival words), else 64-row
    # prefill tiles split over the most workgroups one round holds (at most 8)
    b = F.workspace_size(48, 8192, 8192, 0)
    assert b > 0 and b % (4 * 48 * 8192) != 0
    for (m, N, K), S in (((48, 10240, 8192), 6), ((33, 8200, 8192), 7), ((64, 8192, 28672), 8),
                         ((40, 1000, 8192), 8)):
        assert F.workspace_size(m, N, K, 0) == S * 4 * m * N, (m, N, K)
    # m <= 32 keeps the decode kernel (no split, or planes plus arrival words)
    b = F.workspace_size(24, 10240, 8192, 0)
    assert b == 0 or b % (4 * 24 * 10240) != 0


def test_gemm_rejects_small_or_misaligned_workspace_before_any_hip_call():
    lib = F.lib()
    m, K = 16, 8192
    N = next(n for n in (10240, 8192, 1000) if F.workspace_size(m, n, K, 0) > 0)
    need = F.workspace_size(m, N, K, 0)
    d = ctypes.c_void_p(1 << 20)  # aligned dummy device address; never dereferenced
    assert lib.fp4_gemm(d, d, d, d, m, N, K, 0, None, need, None) == 5
    assert lib.fp4_gemm(d, d, d, d, m, N, K, 0, d, need - 4, None) == 5
    assert lib.fp4_gemm(d, d, d, d, m, N, K, 0, ctypes.c_void_p((1 << 20) + 4), need, None) == 5
    # misaligned operands
    assert lib.fp4_gemm(ctypes.c_void_p((1 << 20) + 2), d, d, d, m, N, K, 0, d, need, None) == 2


def test_noalloc_rejects_problems_beyond_its_scratch():
    # fp4_gemm_noalloc checks the workspace the problem needs against its
    # 64 MiB per-GPU scratch array before any HIP call
    lib = F.lib()
    assert lib.fp4_gemm_noalloc_max_workspace() == 64 << 20
    m, N, K, fmt = 640, 57344, 262144, 0
    assert F.workspace_size(m, N, K, fmt) > lib.fp4_gemm_noalloc_max_workspace()
    d = ctypes.c_void_p(256)   # never dereferenced
    assert lib.fp4_gemm_noalloc(d, d, d, d, m, N, K, fmt, None) == 5      # FP4_ERR_WORKSPACE
    assert lib.fp4_gemm_noalloc(d, d, d, d, 16, 64, 100, 0, None) == 2    # K % 16 != 0
    assert lib.fp4_gemm_noalloc(None, d, d, d, 16, 64, 512, 0, None) == 1
    assert lib.fp4_gemm_noalloc(d, d, d, d, 0, 64, 512, 0, None) == 0     # m == 0: no-op
