"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no attention arithmetic: it only draws random tensors.
Recipe: a CPU ``torch.Generator`` seeded with ``seed`` draws i.i.d. N(0, 1)
fp32 tensors of shape [B, N, H, d] (K and V: [B, N, H_kv, d] for grouped K/V
heads) in the order Q, K, V, dO (dO only when asked), optionally multiplied
by ``gain``, then cast to the requested dtype
(bf16 casts round to nearest even).  The oracle is fed the cast values
upcast to fp64, which is exact for both fp32 and bf16.

FP8 inputs (``make_qkv_fp8``) are the same N(0, 1) draws, quantised per
(batch, head): descale = max|x| / 448 over that head's [N, d] values, and the
code is x / descale cast to OCP E4M3 (torch ``float8_e4m3fn``, round to
nearest even), so each head spans the format's whole range.  The codes (as
bytes) and the fp32 descale factors are the inputs of both sides.
"""

from __future__ import annotations

import numpy as np
import torch

__all__ = ["make_qkv", "make_qkv_fp8", "make_qkv_ramp", "to_f64"]


def make_qkv(B, N, H, d, dtype=torch.bfloat16, seed=0, with_do=False, gain=1.0, H_kv=None):
    """Return a dict with CPU tensors 'q', 'k', 'v' (and 'do') of shape [B,N,H,d];
    with ``H_kv`` (grouped K/V heads) 'k' and 'v' are [B,N,H_kv,d]."""
    g = torch.Generator().manual_seed(int(seed))
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    hkv = H if H_kv is None else H_kv
    out = {}
    for name in names:
        heads = hkv if name in ("k", "v") else H
        t = torch.randn((B, N, heads, d), generator=g, dtype=torch.float32)
        if gain != 1.0:
            t = t * gain
        out[name] = t.to(dtype).contiguous()
    return out


def make_qkv_fp8(B, N, H, d, seed=0, gain=1.0, H_kv=None):
    """Return a dict with uint8 CPU tensors 'q8', 'k8', 'v8' (E4M3 codes,
    [B,N,H,d]; K and V [B,N,H_kv,d]) and fp32 'q_descale' [B,H],
    'k_descale' and 'v_descale' [B,H_kv]."""
    x = make_qkv(B, N, H, d, torch.float32, seed=seed, gain=gain, H_kv=H_kv)
    out = {}
    for name in ("q", "k", "v"):
        t = x[name]
        amax = t.abs().amax(dim=(1, 3))                       # [B, heads]
        descale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        codes = (t / descale[:, None, :, None]).to(torch.float8_e4m3fn)
        out[name + "8"] = codes.view(torch.uint8).contiguous()
        out[name + "_descale"] = descale.to(torch.float32).contiguous()
    return out


def make_qkv_ramp(B, N, H, d, span, seed=0, descending=False, dtype=torch.bfloat16):
    """Inputs whose scores climb (or fall) steadily along the keys.

    Each (batch, head) draws one direction u ~ N(0, I_d); query rows are
    u + 0.25 n and key rows are r_j u + 0.25 n' (n, n' i.i.d. N(0, I_d)) with
    r_j rising linearly from 0 to ``span`` over the keys (falling with
    ``descending``); V is i.i.d. N(0, 1).  Scores q_i . k_j then grow by about
    span |u|^2 from the first key to the last, so a running row maximum is
    raised many times along a row.  Returns CPU tensors 'q', 'k', 'v'."""
    g = torch.Generator().manual_seed(int(seed))
    u = torch.randn((B, 1, H, d), generator=g, dtype=torch.float32)
    r = torch.linspace(0.0, float(span), N, dtype=torch.float32)
    if descending:
        r = r.flip(0)
    q = u + 0.25 * torch.randn((B, N, H, d), generator=g, dtype=torch.float32)
    k = r[None, :, None, None] * u + 0.25 * torch.randn((B, N, H, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, N, H, d), generator=g, dtype=torch.float32)
    return {n: t.to(dtype).contiguous() for n, t in (("q", q), ("k", k), ("v", v))}


def to_f64(t):
    """CPU/GPU torch tensor -> numpy fp64 (exact for fp32 and bf16)."""
    return t.detach().to("cpu", torch.float64).numpy()


def pick_rows(B, H, N, count, seed=1234, include_edges=True):
    """Deterministic sample of (b, h, i) query rows for sampled parity checks.

    Always includes the first and last row of the first and last head, so the
    sample covers the causal edge cases and the ragged tail.
    """
    rng = np.random.default_rng(seed)
    picks = set()
    if include_edges:
        for b, h in ((0, 0), (B - 1, H - 1)):
            for i in (0, 1, N - 2, N - 1):
                if 0 <= i < N:
                    picks.add((b, h, i))
    while len(picks) < count + (8 if include_edges else 0) and len(picks) < B * H * N:
        picks.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(N))))
    return sorted(picks)
