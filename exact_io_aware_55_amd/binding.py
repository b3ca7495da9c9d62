"""Thin ctypes binding of libfa.so (C ABI in include/fa.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs are allocated with torch, and raw device pointers plus the
current HIP stream are handed to the library.  Every arithmetic step runs in
the library's HIP kernels; there is no fallback.  If the shared library is
missing this module raises instead of computing anything.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_bwd_workspace_size", "fa_bwd", "fa_bwd_preprocess",
           "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_dq_stats", "fa_fwd_gqa", "fa_bwd_gqa", "fa_fwd_window",
           "fa_bwd_window", "fa_fwd_fp8", "fa_strerror")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_MISALIGNED = -3
FA_ERR_WORKSPACE = -4
FA_ERR_LAUNCH = -5

_lib = None


def load(path: str = LIB_PATH):
    """Load libfa.so once and declare the C signatures; raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build it with `python -m exact_io_aware_55_amd.build` "
            "(the attention kernels have no other implementation)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd_f32.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, vp, sz, vp]
    lib.fa_bwd_preprocess.restype = i
    lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_dkdv.restype = i
    lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_dq.restype = i
    lib.fa_bwd_dq_stats.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_dq_stats.restype = i
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_gqa.restype = i
    lib.fa_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_gqa.restype = i
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_window.restype = i
    lib.fa_bwd_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_window.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().fa_strerror(code).decode()


def _check(rc: int):
    if rc != FA_OK:
        raise RuntimeError(f"libfa error {rc}: {strerror(rc)}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check_inputs(dtype, *ts):
    shape = ts[0].shape
    if len(shape) != 4:
        raise ValueError("tensors must be [B, N, H, d]")
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t.dtype != dtype:
            raise ValueError(f"expected {dtype}, got {t.dtype}")
        if t.shape != shape:
            raise ValueError("q, k, v (and o, dO) must have the same shape")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, N, H, d]")
    return shape


def _check_gqa(dtype, q_like, kv_like):
    """q-shaped tensors [B,N,H,d] and K/V-shaped tensors [B,N,H_kv,d], H a
    multiple of H_kv.  Returns (B, N, H, H_kv, d)."""
    B, N, H, d = _check_inputs(dtype, *q_like)
    Bk, Nk, Hkv, dk = _check_inputs(dtype, *kv_like)
    if (Bk, Nk, dk) != (B, N, d) or Hkv < 1 or H % Hkv != 0:
        raise ValueError("k and v must be [B, N, H_kv, d] with H a multiple of H_kv")
    return B, N, H, Hkv, d


def _scale(scale, d):
    return float(d) ** -0.5 if scale is None else float(scale)


def forward(q, k, v, causal=False, scale=None, out=None, lse=None, window=None):
    """bf16 forward.  Returns (O [B,N,H,d] bf16, LSE [B,H,N] fp32).

    k and v may have fewer heads than q (grouped-query attention: [B,N,H_kv,d]
    with H a multiple of H_kv); that calls fa_fwd_gqa, else fa_fwd.  ``window``
    (causal sliding window: query i sees keys i - window < j <= i) calls
    fa_fwd_window and implies causal."""
    lib = load()
    B, N, H, Hkv, d = _check_gqa(torch.bfloat16, (q,), (k, v))
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), device=q.device, dtype=torch.float32) if lse is None else lse
    if window is not None:
        _check(lib.fa_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, Hkv, N, d,
                                 _scale(scale, d), int(window), _stream()))
    elif Hkv == H:
        _check(lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
                          _scale(scale, d), int(bool(causal)), _stream()))
    else:
        _check(lib.fa_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, Hkv, N, d,
                              _scale(scale, d), int(bool(causal)), _stream()))
    return o, lse_t


def forward_fp8(q8, k8, v8, q_descale, k_descale, v_descale, causal=False, scale=None, window=None,
                out=None, lse=None):
    """FP8 forward (fa_fwd_fp8).  q8 [B,N,H,d] and k8, v8 [B,N,H_kv,d] are
    uint8 tensors of OCP E4M3 codes; the descales are fp32 [B,H] (Q) and
    [B,H_kv] (K, V).  ``scale`` multiplies the decoded scores (default
    1/sqrt(d)).  Returns (O [B,N,H,d] bf16, LSE [B,H,N] fp32)."""
    lib = load()
    B, N, H, Hkv, d = _check_gqa(torch.uint8, (q8,), (k8, v8))
    for t, heads in ((q_descale, H), (k_descale, Hkv), (v_descale, Hkv)):
        if (not t.is_cuda or t.dtype != torch.float32 or tuple(t.shape) != (B, heads)
                or not t.is_contiguous()):
            raise ValueError("descales must be contiguous fp32 GPU tensors [B, H] (q) and [B, H_kv] (k, v)")
    if window is not None:
        causal = True
    o = torch.empty((B, N, H, d), device=q8.device, dtype=torch.bfloat16) if out is None else out
    lse_t = torch.empty((B, H, N), device=q8.device, dtype=torch.float32) if lse is None else lse
    _check(lib.fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
                          _ptr(o), _ptr(lse_t), B, H, Hkv, N, d, _scale(scale, d), int(bool(causal)),
                          0 if window is None else int(window), _stream()))
    return o, lse_t


def forward_f32(q, k, v, causal=False, scale=None, out=None, lse=None):
    """fp32 forward.  Returns (O [B,N,H,d] fp32, LSE [B,H,N] fp32)."""
    lib = load()
    B, N, H, d = _check_inputs(torch.float32, q, k, v)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), device=q.device, dtype=torch.float32) if lse is None else lse
    _check(lib.fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
                          _scale(scale, d), int(bool(causal)), _stream()))
    return o, lse_t


def bwd_workspace_size(B, H, N, d) -> int:
    return int(load().fa_bwd_workspace_size(B, H, N, d))


def backward(q, k, v, o, do, lse, causal=False, scale=None, workspace=None, out=None, window=None):
    """bf16 backward by recomputation.  Returns (dQ, dK, dV), bf16, shaped like
    q, k and v (grouped-query attention when k and v have fewer heads: then
    fa_bwd_gqa, else fa_bwd; ``window`` as in :func:`forward`: fa_bwd_window)."""
    lib = load()
    B, N, H, Hkv, d = _check_gqa(torch.bfloat16, (q, o, do), (k, v))
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [B, H, N]")
    need = bwd_workspace_size(B, H, N, d)
    ws = torch.empty(need, device=q.device, dtype=torch.uint8) if workspace is None else workspace
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
    if window is not None:
        _check(lib.fa_bwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                                 _ptr(dk), _ptr(dv), B, H, Hkv, N, d, _scale(scale, d), int(window),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    elif Hkv == H:
        _check(lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                          _ptr(dv), B, H, N, d, _scale(scale, d), int(bool(causal)), _ptr(ws),
                          ws.numel() * ws.element_size(), _stream()))
    else:
        _check(lib.fa_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                              _ptr(dk), _ptr(dv), B, H, Hkv, N, d, _scale(scale, d), int(bool(causal)),
                              _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return dq, dk, dv


def backward_steps(q, k, v, o, do, lse, causal=False, scale=None, workspace=None, out=None,
                   preprocess=False):
    """The same backward as :func:`backward`, issued as separate C-ABI steps.

    Returns ((dQ, dK, dV), calls) where ``calls`` is a list of zero-argument
    callables that enqueue the steps again on the current stream, for timing:
    (dQ with the row statistics, dK/dV), the order fa_bwd runs; with
    ``preprocess`` the three-step order (preprocess, dK/dV, dQ)."""
    lib = load()
    B, N, H, d = _check_inputs(torch.bfloat16, q, k, v, o, do)
    need = bwd_workspace_size(B, H, N, d)
    ws = torch.empty(need, device=q.device, dtype=torch.uint8) if workspace is None else workspace
    dq, dk, dv = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if out is None else out
    nbytes = ws.numel() * ws.element_size()
    sc = _scale(scale, d)
    c = int(bool(causal))
    dkdv = lambda: _check(lib.fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv),
                                          B, H, N, d, sc, c, _ptr(ws), nbytes, _stream()))
    if preprocess:
        calls = [
            lambda: _check(lib.fa_bwd_preprocess(_ptr(o), _ptr(do), _ptr(lse), B, H, N, d, _ptr(ws),
                                                 nbytes, _stream())),
            dkdv,
            lambda: _check(lib.fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), B, H, N, d, sc,
                                         c, _ptr(ws), nbytes, _stream())),
        ]
    else:
        calls = [
            lambda: _check(lib.fa_bwd_dq_stats(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                               _ptr(dq), B, H, N, d, sc, c, _ptr(ws), nbytes, _stream())),
            dkdv,
        ]
    for call in calls:
        call()
    return (dq, dk, dv), calls
