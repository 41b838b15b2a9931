"""fp4_gemm_noalloc (the entry point for callers that cannot allocate) against
fp4_gemm, through the C ABI: the same kernels on the same inputs must give
the same bits, and the oracle's tolerance, on two calls in a row whose second
problem is smaller (the per-GPU scratch array keeps the first call's
contents), for a decode K split (partials and arrival words in the scratch),
a prefill K split (partials reduced by a second kernel; also the 64-row tiles
33 <= m <= 64 takes on narrower layers and the 256-row tiles of a long-K layer
at m = 129) and a problem with no split."""

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


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _both(p):
    """(fp4_gemm output bits, fp4_gemm_noalloc output bits) for problem p."""
    wq, sq = F.upload(*F.repack(p.codes, p.scales, p.N, p.K, p.fmt))
    A = torch.from_numpy(np.ascontiguousarray(p.a_bits).view(np.int16)).cuda().view(torch.bfloat16)
    ref = torch.full((p.m, p.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = torch.full((p.m, p.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    need = F.workspace_size(p.m, p.N, p.K, p.fmt)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    stream = F._stream_handle(None)
    lib = F.lib()
    st = lib.fp4_gemm(F._dev_ptr(A), F._dev_ptr(wq), F._dev_ptr(sq), F._dev_ptr(ref), p.m, p.N, p.K, p.fmt,
                      F._dev_ptr(ws), need, stream)
    F._check(st, "fp4_gemm")
    st = lib.fp4_gemm_noalloc(F._dev_ptr(A), F._dev_ptr(wq), F._dev_ptr(sq), F._dev_ptr(out), p.m, p.N, p.K,
                              p.fmt, stream)
    F._check(st, "fp4_gemm_noalloc")
    torch.cuda.synchronize()
    return _bits(ref), _bits(out)


@pytest.mark.parametrize("first,second", [
    ((16, 10240, 8192, 0), (16, 1000, 8192, 0)),        # decode, K split finished in-kernel, then a smaller one
    ((256, 8192, 8192, 0), (100, 520, 2048, 1)),        # prefill K split (reduce kernel), then smaller
    ((16, 8192, 28672, 1), (7, 8200, 8192, 0)),         # down-shaped MXFP4 split, then a ragged NVFP4 one
    ((48, 10240, 4096, 0), (40, 8200, 2048, 1)),        # 64-row prefill tiles with a K split (33 <= m <= 64)
    ((129, 8192, 28672, 0), (256, 32784, 512, 1)),      # 256-row prefill tiles with a K split, then without
])
def test_noalloc_matches_gemm_on_two_calls(first, second):
    for i, (m, N, K, fmt) in enumerate((first, second)):
        print("[case] noalloc", i, m, N, K, fmt, F.workspace_size(m, N, K, fmt), flush=True)
        assert F.workspace_size(m, N, K, fmt) <= F.lib().fp4_gemm_noalloc_max_workspace()
        p = synth.make_random(m, N, K, fmt, seed=900 + 7 * m + N + K + fmt)
        ref, got = _both(p)
        assert np.array_equal(ref, got), f"call {i}: fp4_gemm_noalloc differs from fp4_gemm"
        rows = np.unique(np.concatenate([np.arange(min(N, 48)), np.arange(max(0, N - 48), N),
                                         np.arange(0, N, 37)]))
        y_ref, bound = oracle.gemm_reference(p.a_bits, p.codes[rows], p.scales[rows], K, fmt)
        assert oracle.check_tolerance(got[:, rows], y_ref, bound).all()

