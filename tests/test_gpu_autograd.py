"""binding.attention as a torch autograd operation: its output and the
gradients torch's autograd returns for q, k and v are exactly those of the
explicit forward and backward calls (the same kernels), for plain, causal,
grouped-query and sliding-window attention, and they reach the oracle's
gradients within the bf16 lines."""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_55_amd import binding, inputs
from parity import max_abs, rel_l2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("kind", ["plain", "causal", "gqa", "window"])
def test_autograd_matches_the_explicit_calls(gpu_lib, kind):
    B, N, H, d = 2, 300, 4, 64
    hkv = 2 if kind == "gqa" else H
    causal = kind in ("causal", "gqa")
    window = 50 if kind == "window" else None
    print(f"\n[autograd] {kind} B{B} H{H} Hkv{hkv} N{N} d{d}", flush=True)
    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=61, with_do=True, H_kv=hkv)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = binding.attention(qa, ka, va, causal=causal, window=window)
    o.backward(do)
    o_ref, lse = binding.forward(q, k, v, causal=causal or window is not None, window=window)
    grads = binding.backward(q, k, v, o_ref, do, lse, causal=causal or window is not None, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for got, ref, name in zip((qa.grad, ka.grad, va.grad), grads, ("dq", "dk", "dv")):
        assert torch.equal(got, ref), name


def test_autograd_gradients_reach_the_oracle(gpu_lib):
    """A scalar loss through binding.attention: the gradients torch returns
    match the oracle's backward of the same loss on every head."""
    B, N, H, d = 1, 256, 2, 128
    print(f"\n[autograd] oracle B{B} H{H} N{N} d{d} causal", flush=True)
    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=62, with_do=True)
    q, k, v = (x[n].to(DEV).requires_grad_(True) for n in ("q", "k", "v"))
    w = x["do"].to(DEV)
    loss = (binding.attention(q, k, v, causal=True).float() * w.float()).sum()
    loss.backward()
    torch.cuda.synchronize()
    qn, kn, vn, wn = (inputs.to_f64(x[n]) for n in ("q", "k", "v", "do"))
    for h in range(H):
        ref = oracle.head_backward(qn[0, :, h], kn[0, :, h], vn[0, :, h], wn[0, :, h], d ** -0.5, True)
        for got, r, name in zip((q.grad, k.grad, v.grad), ref, ("dq", "dk", "dv")):
            g = inputs.to_f64(got)[0, :, h]
            assert max_abs(g, r) <= 2e-2 and rel_l2(g, r) <= 5e-3, (name, h)
