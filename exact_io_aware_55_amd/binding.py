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
SYNC_LIB_PATH = os.path.join(_HERE, "libfa_sync.so")   # synchronisation check build

EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_bwd_workspace_size", "fa_bwd", "fa_bwd_preprocess",
           "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_dq_stats", "fa_fwd_gqa", "fa_bwd_gqa", "fa_fwd_window",
           "fa_bwd_window", "fa_fwd_fp8", "fa_bwd_noalloc", "fa_bwd_noalloc_max_workspace", "fa_merge",
           "fa_calibrate_mfma", "fa_probe_mfma", "fa_strerror")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_MISALIGNED = -3
FA_ERR_WORKSPACE = -4
FA_ERR_LAUNCH = -5
FA_ERR_SCRATCH = -6

_lib = None


def load(path: str = LIB_PATH):
    """Load libfa.so once and declare the C signatures; raises if absent."""
    global _lib
    if _lib is None:
        _lib = open_library(path)
    return _lib


def open_library(path: str):
    """A library with the C ABI of include/fa.h (libfa.so or its
    synchronisation check build libfa_sync.so), signatures declared; raises
    if absent.  Not cached: load() keeps the one the functions below use."""
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
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc_max_workspace.argtypes = []
    lib.fa_bwd_noalloc_max_workspace.restype = sz
    lib.fa_merge.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
    lib.fa_merge.restype = i
    lib.fa_calibrate_mfma.argtypes = [vp, i, i, i, i, vp]
    lib.fa_calibrate_mfma.restype = i
    lib.fa_probe_mfma.argtypes = [i, vp, vp, vp, i, i, vp]
    lib.fa_probe_mfma.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
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


def _on_device(t):
    return t.is_cuda


def _need(t, name, dtype, shape, device):
    """A caller-supplied tensor the kernels read or write: it must be a
    contiguous tensor of ``dtype`` and ``shape`` on ``device``.  The C ABI
    sees only a raw pointer, so a host tensor or a short buffer would reach
    the kernels unchecked."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if not _on_device(t) or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _need_bytes(t, name, nbytes, device):
    """A workspace: a contiguous device tensor of at least ``nbytes`` bytes."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if not _on_device(t) or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, {nbytes} needed")
    return t


def _check_inputs(dtype, *ts):
    shape = ts[0].shape
    if len(shape) != 4:
        raise ValueError("tensors must be [B, N, H, d]")
    for t in ts:
        if not _on_device(t):
            raise ValueError("tensors must be on the GPU")
        if t.device != ts[0].device:
            raise ValueError("tensors must be on one device")
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
    if kv_like[0].device != q_like[0].device:
        raise ValueError("tensors must be on one device")
    if (Bk, Nk, dk) != (B, N, d) or Hkv < 1 or H % Hkv != 0:
        raise ValueError("k and v must be [B, N, H_kv, d] with H a multiple of H_kv")
    return B, N, H, Hkv, d


def _outputs(out, like, names):
    """Caller-supplied output tensors (or None: allocate like ``like``)."""
    if out is None:
        return tuple(torch.empty_like(t) for t in like)
    if len(out) != len(like):
        raise ValueError(f"out must hold {len(like)} tensors")
    return tuple(_need(o, n, t.dtype, t.shape, t.device) for o, t, n in zip(out, like, names))


def _lse_out(lse, B, H, N, device):
    if lse is None:
        return torch.empty((B, H, N), device=device, dtype=torch.float32)
    return _need(lse, "lse", torch.float32, (B, H, N), device)


def _workspace(workspace, B, H, N, d, device):
    need = bwd_workspace_size(B, H, N, d)
    if workspace is None:
        return torch.empty(need, device=device, dtype=torch.uint8)
    return _need_bytes(workspace, "workspace", need, device)


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
    (o,) = _outputs(None if out is None else (out,), (q,), ("out",))
    lse_t = _lse_out(lse, B, H, N, q.device)
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
    for t, name, heads in ((q_descale, "q_descale", H), (k_descale, "k_descale", Hkv),
                           (v_descale, "v_descale", Hkv)):
        _need(t, name, torch.float32, (B, heads), q8.device)
    if window is not None:
        causal = True
    if out is None:
        o = torch.empty((B, N, H, d), device=q8.device, dtype=torch.bfloat16)
    else:
        o = _need(out, "out", torch.bfloat16, (B, N, H, d), q8.device)
    lse_t = _lse_out(lse, B, H, N, q8.device)
    _check(lib.fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
                          _ptr(o), _ptr(lse_t), B, H, Hkv, N, d, _scale(scale, d), int(bool(causal)),
                          0 if window is None else int(window), _stream()))
    return o, lse_t


def forward_f32(q, k, v, causal=False, scale=None, out=None, lse=None):
    """fp32 forward.  Returns (O [B,N,H,d] fp32, LSE [B,H,N] fp32)."""
    lib = load()
    B, N, H, d = _check_inputs(torch.float32, q, k, v)
    (o,) = _outputs(None if out is None else (out,), (q,), ("out",))
    lse_t = _lse_out(lse, B, H, N, q.device)
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
    _need(lse, "lse", torch.float32, (B, H, N), q.device)
    ws = _workspace(workspace, B, H, N, d, q.device)
    dq, dk, dv = _outputs(out, (q, k, v), ("dq", "dk", "dv"))
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


def backward_noalloc(q, k, v, o, do, lse, causal=False, scale=None, out=None):
    """The backward of :func:`backward` through fa_bwd_noalloc, whose
    workspace is the library's static scratch array (no device allocation
    inside the library; the outputs are allocated here unless ``out`` gives
    them).  Multi-head attention only."""
    lib = load()
    B, N, H, d = _check_inputs(torch.bfloat16, q, k, v, o, do)
    _need(lse, "lse", torch.float32, (B, H, N), q.device)
    dq, dk, dv = _outputs(out, (q, k, v), ("dq", "dk", "dv"))
    _check(lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                              _ptr(dv), B, H, N, d, _scale(scale, d), int(bool(causal)), _stream()))
    return dq, dk, dv


def _overlap(a, b):
    """True if two tensors share any byte of memory without being the same
    buffer (a partial overlap)."""
    a0, b0 = a.data_ptr(), b.data_ptr()
    a1, b1 = a0 + a.numel() * a.element_size(), b0 + b.numel() * b.element_size()
    return a0 < b1 and b0 < a1 and not (a0 == b0 and a1 == b1)


def merge(o_a, lse_a, o_b, lse_b, out=None, lse_out=None):
    """Attention over the union of two disjoint key ranges from the results
    over each (fa_merge): O = exp(LSE_a - L) O_a + exp(LSE_b - L) O_b with
    L = log(exp(LSE_a) + exp(LSE_b)).  o_a, o_b: bf16 [B,N,H,d]; lse_a, lse_b:
    fp32 [B,H,N].  ``out`` may be o_a or o_b and ``lse_out`` lse_a or lse_b
    (accumulation in place).  Returns (O, LSE)."""
    lib = load()
    B, N, H, d = _check_inputs(torch.bfloat16, o_a, o_b)
    dev = o_a.device
    _need(lse_a, "lse_a", torch.float32, (B, H, N), dev)
    _need(lse_b, "lse_b", torch.float32, (B, H, N), dev)
    o = torch.empty_like(o_a) if out is None else _need(out, "out", torch.bfloat16, o_a.shape, dev)
    lse = _lse_out(lse_out, B, H, N, dev)
    for t, srcs in ((o, (o_a, o_b)), (lse, (lse_a, lse_b))):
        if any(_overlap(t, x) for x in srcs):
            raise ValueError("an output may be one of the inputs but must not partly overlap one")
    _check(lib.fa_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(lse), B, H, N, d,
                        _stream()))
    return o, lse


def calibrate_mfma(n_workgroups, waves=4, iters=4096, mode=0, out=None):
    """Launch the matrix-core calibration kernel once on the current stream
    (fa_calibrate_mfma; ``mode`` 0 constant operands, 1 random operands, 2 and
    3 random plus 2 or 4 vector instructions per MFMA, 4 random with the A
    operand from LDS, 5 mode 4 plus three FMAs and one exp2 per MFMA, 6 mode
    5 with each LDS read feeding two MFMAs, 7 mode 4 plus four FMAs and one
    exp2 per two MFMAs).  Returns (checksum tensor, flops of the launch)."""
    lib = load()
    dev = torch.device("cuda", torch.cuda.current_device())
    n = n_workgroups * 64 * waves
    o = torch.empty(n, device=dev, dtype=torch.float32) if out is None else _need(out, "out", torch.float32,
                                                                                   (n,), dev)
    _check(lib.fa_calibrate_mfma(_ptr(o), n_workgroups, waves, iters, mode, _stream()))
    return o, n_workgroups * waves * iters * 16 * 32768


def probe_mfma(a, b, fp8=False):
    """C = A B^T per 32 x 32 tile on the matrix core (fa_probe_mfma): a, b
    are [tiles, 32, k] GPU tensors (bf16, or uint8 E4M3 codes with fp8).
    Returns C [tiles, 32, 32] fp32."""
    lib = load()
    dt = torch.uint8 if fp8 else torch.bfloat16
    if a.dim() != 3 or a.shape[1] != 32:
        raise ValueError("a must be [tiles, 32, k]")
    _need(a, "a", dt, a.shape, a.device)
    _need(b, "b", dt, a.shape, a.device)
    c = torch.empty((a.shape[0], 32, 32), device=a.device, dtype=torch.float32)
    _check(lib.fa_probe_mfma(int(bool(fp8)), _ptr(a), _ptr(b), _ptr(c), a.shape[0], a.shape[2], _stream()))
    return c


def backward_steps(q, k, v, o, do, lse, causal=False, scale=None, workspace=None, out=None,
                   preprocess=False):
    """The same backward as :func:`backward`, issued as separate C-ABI steps.

    Returns ((dQ, dK, dV), calls) where ``calls`` is a list of zero-argument
    callables that enqueue the steps again on the current stream, for timing:
    (dQ with the row statistics, dK/dV), the order fa_bwd runs; with
    ``preprocess`` the three-step order (preprocess, dK/dV, dQ)."""
    lib = load()
    B, N, H, d = _check_inputs(torch.bfloat16, q, k, v, o, do)
    _need(lse, "lse", torch.float32, (B, H, N), q.device)
    ws = _workspace(workspace, B, H, N, d, q.device)
    dq, dk, dv = _outputs(out, (q, k, v), ("dq", "dk", "dv"))
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


class _Attention(torch.autograd.Function):
    """forward / backward of the library as one autograd node: O is
    returned; the backward consumes O and LSE saved from the forward."""

    @staticmethod
    def forward(ctx, q, k, v, causal, scale, window):
        o, lse = forward(q, k, v, causal=causal, scale=scale, window=window)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale, ctx.window = causal, scale, window
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, do.contiguous(), lse, causal=ctx.causal, scale=ctx.scale,
                              window=ctx.window)
        return dq, dk, dv, None, None, None


def attention(q, k, v, causal=False, scale=None, window=None):
    """O of :func:`forward` as a differentiable torch operation: gradients
    with respect to q, k and v come from :func:`backward` (grouped-query
    attention and sliding windows as there).  bf16 [B,N,H,d] tensors."""
    return _Attention.apply(q, k, v, bool(causal) or window is not None, scale, window)

