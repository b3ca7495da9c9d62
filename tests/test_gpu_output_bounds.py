"""Every entry point writes all of its outputs and nothing around them.

Each output (and the backward's workspace) is a view into a larger buffer whose
guard regions, before and after it, hold a fixed bit pattern (a NaN payload no
kernel produces from finite inputs).  With B = 1 and a ragged N, a row stored
past N, or a head or feature offset past the last one, lands in the trailing
guard.  The guards must come back bit for bit, and no output element may still
hold the pattern (every element was written).
"""

import math

import pytest
import torch

from exact_io_aware_55_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD = 4096                     # elements each side: views stay 256-byte aligned
FILL = {torch.bfloat16: (torch.int16, 0x7FA5), torch.float32: (torch.int32, 0x7FA5A5A5),
        torch.uint8: (torch.uint8, 0xA5)}


class Guarded:
    """A tensor of `shape` inside a buffer with GUARD filled elements each side."""

    def __init__(self, shape, dtype):
        self.n = math.prod(shape)
        self.dtype = dtype
        self.buf = torch.empty(2 * GUARD + self.n, dtype=dtype, device=DEV)
        itype, bits = FILL[dtype]
        self.buf.view(itype).fill_(bits)
        self.t = self.buf[GUARD:GUARD + self.n].view(shape)

    def check(self, name, all_written=True):
        itype, bits = FILL[self.dtype]
        raw = self.buf.view(itype)
        before = int((raw[:GUARD] != bits).sum())
        after = int((raw[GUARD + self.n:] != bits).sum())
        assert before == 0 and after == 0, f"{name}: {before} elements before and {after} after it changed"
        if all_written:
            left = int((raw[GUARD:GUARD + self.n] == bits).sum())
            assert left == 0, f"{name}: {left} elements never written"


def qkv(N, H, d, Hkv=None, seed=0):
    x = inputs.make_qkv(1, N, H, d, seed=seed, with_do=True, H_kv=Hkv)
    return {k: v.to(DEV) for k, v in x.items()}


SHAPES = [(77, 64), (333, 128), (200, 64), (77, 128)]


@pytest.mark.parametrize("N,d", SHAPES)
@pytest.mark.parametrize("kind", ["plain", "causal", "window", "gqa"])
def test_forward_and_backward_stay_in_bounds(gpu_lib, N, d, kind):
    H, Hkv = (4, 2) if kind == "gqa" else (3, 3)
    x = qkv(N, H, d, Hkv if kind == "gqa" else None)
    causal = kind in ("causal", "gqa")
    window = 40 if kind == "window" else None
    o = Guarded((1, N, H, d), torch.bfloat16)
    lse = Guarded((1, H, N), torch.float32)
    gpu_lib.forward(x["q"], x["k"], x["v"], causal=causal, window=window, out=o.t, lse=lse.t)
    torch.cuda.synchronize()
    o.check("O")
    lse.check("LSE")

    ws = Guarded((gpu_lib.bwd_workspace_size(1, H, N, d),), torch.uint8)
    dq = Guarded((1, N, H, d), torch.bfloat16)
    dk = Guarded((1, N, Hkv, d), torch.bfloat16)
    dv = Guarded((1, N, Hkv, d), torch.bfloat16)
    gpu_lib.backward(x["q"], x["k"], x["v"], o.t, x["do"], lse.t, causal=causal, window=window,
                     workspace=ws.t, out=(dq.t, dk.t, dv.t))
    torch.cuda.synchronize()
    for g, name in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
        g.check(name)
    ws.check("workspace", all_written=False)


@pytest.mark.parametrize("N,d", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_variants_stay_in_bounds(gpu_lib, N, d, causal):
    H = 3
    x = qkv(N, H, d, seed=1)
    o, lse = gpu_lib.forward(x["q"], x["k"], x["v"], causal=causal)
    for how in ("noalloc", "steps"):
        dq, dk, dv = (Guarded((1, N, H, d), torch.bfloat16) for _ in range(3))
        out = (dq.t, dk.t, dv.t)
        if how == "noalloc":
            gpu_lib.backward_noalloc(x["q"], x["k"], x["v"], o, x["do"], lse, causal=causal, out=out)
        else:
            ws = Guarded((gpu_lib.bwd_workspace_size(1, H, N, d),), torch.uint8)
            gpu_lib.backward_steps(x["q"], x["k"], x["v"], o, x["do"], lse, causal=causal, workspace=ws.t,
                                   out=out, preprocess=True)
        torch.cuda.synchronize()
        for g, name in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
            g.check(f"{how} {name}")
        if how == "steps":
            ws.check("steps workspace", all_written=False)


@pytest.mark.parametrize("N,d", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_stays_in_bounds(gpu_lib, N, d, causal):
    H, Hkv = 4, 2
    x = {k: v.to(DEV) for k, v in inputs.make_qkv_fp8(1, N, H, d, seed=2, H_kv=Hkv).items()}
    o = Guarded((1, N, H, d), torch.bfloat16)
    lse = Guarded((1, H, N), torch.float32)
    gpu_lib.forward_fp8(x["q8"], x["k8"], x["v8"], x["q_descale"], x["k_descale"], x["v_descale"],
                        causal=causal, out=o.t, lse=lse.t)
    torch.cuda.synchronize()
    o.check("FP8 O")
    lse.check("FP8 LSE")


@pytest.mark.parametrize("N,d", SHAPES)
def test_f32_forward_and_merge_stay_in_bounds(gpu_lib, N, d):
    H = 3
    x = inputs.make_qkv(1, N, H, d, torch.float32, seed=3)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o = Guarded((1, N, H, d), torch.float32)
    lse = Guarded((1, H, N), torch.float32)
    gpu_lib.forward_f32(q, k, v, causal=True, out=o.t, lse=lse.t)
    torch.cuda.synchronize()
    o.check("fp32 O")
    lse.check("fp32 LSE")

    # two partial results to combine (their meaning does not matter here)
    y, z = qkv(N, H, d, seed=4), qkv(N, H, d, seed=5)
    o_a, lse_a = gpu_lib.forward(y["q"], y["k"], y["v"])
    o_b, lse_b = gpu_lib.forward(z["q"], z["k"], z["v"], causal=True)
    om = Guarded((1, N, H, d), torch.bfloat16)
    lm = Guarded((1, H, N), torch.float32)
    gpu_lib.merge(o_a, lse_a, o_b, lse_b, out=om.t, lse_out=lm.t)
    torch.cuda.synchronize()
    om.check("merged O")
    lm.check("merged LSE")
