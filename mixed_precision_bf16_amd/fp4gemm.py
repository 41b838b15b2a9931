"""ctypes binding of ``libfp4gemm.so`` (argument marshalling only).

Every step of the GEMM runs in the HIP library; this module turns NumPy /
PyTorch buffers into pointers and status codes into exceptions.  PyTorch is
used for device memory and the current HIP stream.  There is no fallback: if
the library is missing or the device is not gfx950, calls raise.
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np

from . import build as _build

NVFP4 = 0
MXFP4 = 1
GROUP = {NVFP4: 16, MXFP4: 32}

_c_i64 = ctypes.c_int64
_c_vp = ctypes.c_void_p
_c_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/fp4gemm.h
_SIGNATURES = {
    "fp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp4_repack_size": (ctypes.c_int, [_c_i64, _c_i64, ctypes.c_int, ctypes.POINTER(_c_sz), ctypes.POINTER(_c_sz)]),
    "fp4_repack": (ctypes.c_int, [_c_vp, _c_vp, _c_i64, _c_i64, ctypes.c_int, _c_vp, _c_vp]),
    "fp4_unpack": (ctypes.c_int, [_c_vp, _c_vp, _c_i64, _c_i64, ctypes.c_int, _c_vp, _c_vp]),
    "fp4_gemm_workspace_size": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, ctypes.c_int, ctypes.POINTER(_c_sz)]),
    "fp4_gemm": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_vp, _c_sz,
                                _c_vp]),
    "fp4_gemm_noalloc": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_vp]),
    "fp4_gemm_noalloc_max_workspace": (ctypes.c_size_t, []),
    "fp4_gemm_f16": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_vp,
                                    _c_sz, _c_vp]),
    "fp4_dequant": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, ctypes.c_int, _c_vp]),
    "fp4_dequant_f16": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, ctypes.c_int, _c_vp]),
    "fp4_gemm_ex": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_float, _c_vp, _c_sz, _c_vp]),
    "fp4_quantize": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, ctypes.c_int, ctypes.c_float, _c_vp]),
    "fp4_native_repack_size": (ctypes.c_int, [_c_i64, _c_i64, ctypes.POINTER(_c_sz), ctypes.POINTER(_c_sz)]),
    "fp4_native_repack": (ctypes.c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp]),
    "fp4_native_unpack": (ctypes.c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp]),
    "fp4_gemm_native_workspace_size": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fp4_gemm_native": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, ctypes.c_float, _c_vp,
                                       _c_sz, _c_vp]),
    "fp4_moe_gemm": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64,
                                    _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_vp]),
}

STATUS = {0: "FP4_OK", 1: "FP4_ERR_NULL", 2: "FP4_ERR_SHAPE", 3: "FP4_ERR_FORMAT", 4: "FP4_ERR_VALUE",
          5: "FP4_ERR_WORKSPACE", 6: "FP4_ERR_DEVICE", 7: "FP4_ERR_HIP"}


class Fp4Error(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib().fp4_status_string(status).decode()
        super().__init__(f"{what}: {STATUS.get(status, status)} ({msg})")


_LIB = None


def lib_path() -> str:
    return _build.LIB_PATH


def lib():
    """Load the library (building it once if it was never built)."""
    global _LIB
    if _LIB is None:
        path = _build.ensure_built()
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def header_functions():
    """Names of the functions declared in include/fp4gemm.h."""
    hdr = os.path.join(_build.ROOT, "include", "fp4gemm.h")
    text = open(hdr).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(fp4_\w+)\s*\(", text, re.M)))


def _check(status: int, what: str):
    if status != 0:
        raise Fp4Error(status, what)


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(_c_vp)


# ------------------------------------------------------------------ host API
def repack_size(N: int, K: int, fmt: int):
    wq, sq = _c_sz(), _c_sz()
    _check(lib().fp4_repack_size(N, K, fmt, ctypes.byref(wq), ctypes.byref(sq)), "fp4_repack_size")
    return wq.value, sq.value


def repack(codes: np.ndarray, scales: np.ndarray, N: int, K: int, fmt: int):
    """Canonical codes [N][K/2] and scales [N][K/G] (uint8, host) -> packed (wq, sq)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    if codes.size != N * (K // 2) or scales.size != N * (K // GROUP.get(fmt, 1)):
        raise ValueError("codes / scales do not match N, K, format")
    nw, ns = repack_size(N, K, fmt)
    wq = np.empty(nw, dtype=np.uint8)
    sq = np.empty(ns, dtype=np.uint8)
    _check(lib().fp4_repack(_np_ptr(codes), _np_ptr(scales), N, K, fmt, _np_ptr(wq), _np_ptr(sq)), "fp4_repack")
    return wq, sq


def unpack(wq: np.ndarray, sq: np.ndarray, N: int, K: int, fmt: int):
    """Packed (wq, sq) -> canonical (codes [N][K/2], scales [N][K/G])."""
    nw, ns = repack_size(N, K, fmt)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    sq = np.ascontiguousarray(sq, dtype=np.uint8)
    if wq.size != nw or sq.size != ns:
        raise ValueError("packed arrays have the wrong size")
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // GROUP[fmt]), dtype=np.uint8)
    _check(lib().fp4_unpack(_np_ptr(wq), _np_ptr(sq), N, K, fmt, _np_ptr(codes), _np_ptr(scales)), "fp4_unpack")
    return codes, scales


def workspace_size(m: int, N: int, K: int, fmt: int) -> int:
    b = _c_sz()
    _check(lib().fp4_gemm_workspace_size(m, N, K, fmt, ctypes.byref(b)), "fp4_gemm_workspace_size")
    return b.value


# ---------------------------------------------------------------- device API
def _dev_ptr(t):
    return _c_vp(t.data_ptr()) if t is not None else _c_vp(0)


def _on_device_of(ref, **tensors):
    """Raise ValueError unless every given tensor (None allowed) is a CUDA
    tensor on ref's device: a host pointer handed to a kernel would fault."""
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != ref.device):
            raise ValueError(f"{name} must be a CUDA tensor on {ref.device}")


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return _c_vp(stream.cuda_stream)


def new_workspace(m: int, N: int, K: int, fmt: int, device="cuda"):
    """A zero-filled workspace for fp4_gemm of this shape (None if none is needed)."""
    import torch
    nbytes = workspace_size(m, N, K, fmt)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def gemm(A, wq, sq, N: int, K: int, fmt: int, out=None, workspace=None, stream=None, alpha: float = 1.0):
    """Y = alpha * A . dequant(W)^T.  A: bfloat16 (fp4_gemm) or float16
    (fp4_gemm_f16) CUDA [m][K]; wq, sq: uint8 CUDA (packed).  alpha != 1 goes
    through fp4_gemm_ex.  Returns (or fills) a tensor [m][N] of A's dtype."""
    import torch
    if A.dtype not in (torch.bfloat16, torch.float16) or A.dim() != 2 or not A.is_cuda or not A.is_contiguous():
        raise ValueError("A must be a contiguous 2-D bfloat16 or float16 CUDA tensor")
    if A.shape[1] != K:
        raise ValueError("A must have K columns")
    for t in (wq, sq):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("wq / sq must be contiguous uint8 CUDA tensors")
    nw, ns = repack_size(N, K, fmt)
    if wq.numel() != nw or sq.numel() != ns:
        raise ValueError("packed weight tensors have the wrong size")
    m = A.shape[0]
    if out is None:
        out = torch.empty((m, N), dtype=A.dtype, device=A.device)
    elif out.shape != (m, N) or out.dtype != A.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor [m][N] of A's dtype")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    _on_device_of(A, wq=wq, sq=sq, out=out, workspace=workspace)
    wsb = workspace_size(m, N, K, fmt)
    if wsb and workspace is None:
        workspace = torch.zeros(wsb, dtype=torch.uint8, device=A.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if alpha != 1.0:
        act = 0 if A.dtype == torch.bfloat16 else 1
        _check(lib().fp4_gemm_ex(_dev_ptr(A), _dev_ptr(wq), _dev_ptr(sq), _dev_ptr(out), m, N, K, fmt, act, alpha,
                                 _dev_ptr(workspace), ws_bytes, _stream_handle(stream)), "fp4_gemm_ex")
        return out
    fn = lib().fp4_gemm if A.dtype == torch.bfloat16 else lib().fp4_gemm_f16
    _check(fn(_dev_ptr(A), _dev_ptr(wq), _dev_ptr(sq), _dev_ptr(out), m, N, K, fmt, _dev_ptr(workspace), ws_bytes,
              _stream_handle(stream)), "fp4_gemm")
    return out


def gemm_noalloc(A, wq, sq, N: int, K: int, fmt: int, out, stream=None):
    """fp4_gemm_noalloc: Y = A . dequant(W)^T with the library's own per-GPU
    scratch instead of a workspace (nothing is allocated; `out`, a contiguous
    bfloat16 CUDA tensor [m][N], must be given)."""
    import torch
    if A.dtype != torch.bfloat16 or A.dim() != 2 or not A.is_cuda or not A.is_contiguous() or A.shape[1] != K:
        raise ValueError("A must be a contiguous bfloat16 CUDA tensor [m][K]")
    for t in (wq, sq):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("wq / sq must be contiguous uint8 CUDA tensors")
    nw, ns = repack_size(N, K, fmt)
    if wq.numel() != nw or sq.numel() != ns:
        raise ValueError("packed weight tensors have the wrong size")
    m = A.shape[0]
    if out is None or out.shape != (m, N) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor [m][N]")
    _on_device_of(A, wq=wq, sq=sq, out=out)
    _check(lib().fp4_gemm_noalloc(_dev_ptr(A), _dev_ptr(wq), _dev_ptr(sq), _dev_ptr(out), m, N, K, fmt,
                                  _stream_handle(stream)), "fp4_gemm_noalloc")
    return out


def quantize(W, fmt: int, alpha: float = 1.0, stream=None):
    """fp4_quantize: BF16 CUDA weights [N][K] -> (codes uint8 [N][K/2], scales
    uint8 [N][K/G]) on the device, in the source order repack() takes."""
    import torch
    if W.dtype != torch.bfloat16 or W.dim() != 2 or not W.is_cuda or not W.is_contiguous():
        raise ValueError("W must be a contiguous 2-D bfloat16 CUDA tensor")
    N, K = W.shape
    G = 16 if fmt == NVFP4 else 32
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scales = torch.empty((N, max(K // G, 1)), dtype=torch.uint8, device=W.device)
    _check(lib().fp4_quantize(_dev_ptr(W), _dev_ptr(codes), _dev_ptr(scales), N, K, fmt, alpha,
                              _stream_handle(stream)), "fp4_quantize")
    return codes, scales


def dequant(wq, sq, N: int, K: int, fmt: int, out=None, stream=None, dtype=None):
    """Weights [N][K] exactly as the GEMM feeds them to the matrix core:
    bfloat16 (default) or float16 (dtype=torch.float16)."""
    import torch
    dtype = torch.bfloat16 if dtype is None else dtype
    if dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("dtype must be torch.bfloat16 or torch.float16")
    for t in (wq, sq):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("wq / sq must be contiguous uint8 CUDA tensors")
    nw, ns = repack_size(N, K, fmt)
    if wq.numel() != nw or sq.numel() != ns:
        raise ValueError("packed weight tensors have the wrong size")
    if out is None:
        out = torch.empty((N, K), dtype=dtype, device=wq.device)
    elif out.shape != (N, K) or out.dtype != dtype or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous CUDA tensor [N][K] of the requested dtype")
    _on_device_of(wq, sq=sq, out=out)
    fn = lib().fp4_dequant if dtype == torch.bfloat16 else lib().fp4_dequant_f16
    _check(fn(_dev_ptr(wq), _dev_ptr(sq), _dev_ptr(out), N, K, fmt, _stream_handle(stream)), "fp4_dequant")
    return out


def upload(wq: np.ndarray, sq: np.ndarray, device="cuda"):
    """Copy packed host arrays to device uint8 tensors."""
    import torch
    return (torch.from_numpy(np.ascontiguousarray(wq)).to(device),
            torch.from_numpy(np.ascontiguousarray(sq)).to(device))


def moe_gemm(A, wq, sq, sorted_ids, expert_offsets, N: int, K: int, fmt: int, E: int, a_div: int, out_rows: int,
             topk_weights=None, out=None, stream=None):
    """Grouped MoE GEMM (fp4_moe_gemm): for each expert e and assignment id in
    sorted_ids[expert_offsets[e]:expert_offsets[e+1]],
    out[id] = w[id] * A[id // a_div] . dequant(W_e)^T.  wq / sq hold the E
    experts' packed weights back to back (each repack_size(N, K, fmt)).  Rows
    of out not listed in sorted_ids are left as they were."""
    import torch
    if A.dtype != torch.bfloat16 or A.dim() != 2 or not A.is_cuda or not A.is_contiguous() or A.shape[1] != K:
        raise ValueError("A must be a contiguous bfloat16 CUDA tensor [a_rows][K]")
    nw, ns = repack_size(N, K, fmt)
    for t, n in ((wq, nw), (sq, ns)):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous() or t.numel() != E * n:
            raise ValueError("wq / sq must be contiguous uint8 CUDA tensors holding E packed experts")
    for t, dt in ((sorted_ids, torch.int32), (expert_offsets, torch.int32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous() or t.dim() != 1:
            raise ValueError("sorted_ids / expert_offsets must be contiguous int32 CUDA vectors")
    if expert_offsets.numel() != E + 1:
        raise ValueError("expert_offsets must have E + 1 entries")
    if topk_weights is not None and (topk_weights.dtype != torch.float32 or not topk_weights.is_cuda
                                     or not topk_weights.is_contiguous() or topk_weights.numel() != out_rows):
        raise ValueError("topk_weights must be a contiguous float32 CUDA vector of out_rows entries")
    if out is None:
        out = torch.zeros((out_rows, N), dtype=torch.bfloat16, device=A.device)
    elif out.shape != (out_rows, N) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor [out_rows][N]")
    _on_device_of(A, wq=wq, sq=sq, sorted_ids=sorted_ids, expert_offsets=expert_offsets,
                  topk_weights=topk_weights, out=out)
    _check(lib().fp4_moe_gemm(_dev_ptr(A), _dev_ptr(wq), _dev_ptr(sq), _dev_ptr(sorted_ids), _dev_ptr(expert_offsets),
                              _dev_ptr(topk_weights), _dev_ptr(out), A.shape[0], a_div, out_rows,
                              sorted_ids.numel(), E, N, K, fmt, _stream_handle(stream)), "fp4_moe_gemm")
    return out


def native_repack(codes, scales, N: int, K: int):
    """fp4_native_repack: canonical MXFP4 codes / scales (host, uint8) -> native
    packed (wq, sq) as CPU uint8 tensors."""
    import numpy as np
    import torch
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    if codes.size != N * K // 2 or scales.size != N * (K // 32):
        raise ValueError("codes / scales have the wrong size")
    nw, ns = native_repack_size(N, K)
    wq = np.empty(nw, np.uint8)
    sq = np.empty(ns, np.uint8)
    _check(lib().fp4_native_repack(codes.ctypes.data_as(_c_vp), scales.ctypes.data_as(_c_vp), N, K,
                                   wq.ctypes.data_as(_c_vp), sq.ctypes.data_as(_c_vp)), "fp4_native_repack")
    return torch.from_numpy(wq), torch.from_numpy(sq)


def native_unpack(wq, sq, N: int, K: int):
    """Inverse of native_repack (host arrays or CPU tensors) -> (codes, scales) numpy."""
    import numpy as np
    wq = np.ascontiguousarray(wq.numpy() if hasattr(wq, "numpy") else wq, dtype=np.uint8)
    sq = np.ascontiguousarray(sq.numpy() if hasattr(sq, "numpy") else sq, dtype=np.uint8)
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, K // 32), np.uint8)
    _check(lib().fp4_native_unpack(wq.ctypes.data_as(_c_vp), sq.ctypes.data_as(_c_vp), N, K,
                                   codes.ctypes.data_as(_c_vp), scales.ctypes.data_as(_c_vp)), "fp4_native_unpack")
    return codes, scales


def native_workspace_size(m: int, N: int, K: int) -> int:
    b = _c_sz()
    _check(lib().fp4_gemm_native_workspace_size(m, N, K, ctypes.byref(b)), "fp4_gemm_native_workspace_size")
    return b.value


def native_repack_size(N: int, K: int):
    wqb, sqb = _c_sz(), _c_sz()
    _check(lib().fp4_native_repack_size(N, K, ctypes.byref(wqb), ctypes.byref(sqb)), "fp4_native_repack_size")
    return wqb.value, sqb.value


def gemm_native(A, wq, sq, N: int, K: int, out=None, workspace=None, stream=None, alpha: float = 1.0):
    """fp4_gemm_native: C = alpha * dequant(quantize_mxfp4(A)) . dequant(W)^T
    with W in the native layout; A bfloat16 CUDA [m][K]; wq / sq uint8 CUDA
    tensors of native_repack_size(N, K) bytes (upload native_repack's CPU
    tensors first)."""
    import torch
    if A.dtype != torch.bfloat16 or A.dim() != 2 or not A.is_cuda or not A.is_contiguous() or A.shape[1] != K:
        raise ValueError("A must be a contiguous bfloat16 CUDA tensor [m][K]")
    nw, ns = native_repack_size(N, K)
    for t, n in ((wq, nw), (sq, ns)):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous() or t.numel() != n:
            raise ValueError("wq / sq must be contiguous uint8 CUDA tensors of native_repack_size(N, K) bytes")
    m = A.shape[0]
    if out is None:
        out = torch.empty((m, N), dtype=torch.bfloat16, device=A.device)
    elif out.shape != (m, N) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor [m][N]")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    _on_device_of(A, wq=wq, sq=sq, out=out, workspace=workspace)
    need = native_workspace_size(m, N, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().fp4_gemm_native(_dev_ptr(A), _dev_ptr(wq), _dev_ptr(sq), _dev_ptr(out), m, N, K, alpha,
                                 _dev_ptr(workspace), ws_bytes, _stream_handle(stream)), "fp4_gemm_native")
    return out
