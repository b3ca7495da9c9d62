"""GPU parity of the forward entry points (fa_fwd, fa_fwd_f32) against the
fp64 oracle, on seeded synthetic inputs, through the C ABI."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_55_amd import inputs, workloads
from parity import assert_f32_close, check_parity, check_rows_forward

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_bf16(lib, x, causal, scale=None):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = lib.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def check_full(lib, B, N, H, d, causal, seed, scale=None):
    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=seed)
    sc = d ** -0.5 if scale is None else scale
    o, lse = run_bf16(lib, x, causal, scale=sc)
    check_parity(x, sc, causal, o=o, lse=lse, what=f"B{B} N{N} H{H} d{d} causal={causal} scale={sc}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 7, 63, 64, 65, 127, 128, 129, 300, 1000])
def test_bf16_small_shapes(gpu_lib, N, d, causal):
    print(f"\n[fwd bf16] N={N} d={d} causal={causal}", flush=True)
    check_full(gpu_lib, 2, N, 3, d, causal, seed=100 + N)


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_scale_edge_cases(gpu_lib, causal):
    """scale = 0 gives the (prefix) mean of V; a negative scale is still exact attention."""
    for sc in (0.0, -0.2, 0.7):
        print(f"\n[fwd bf16] scale={sc} causal={causal}", flush=True)
        check_full(gpu_lib, 1, 200, 2, 64, causal, seed=7, scale=sc)
        check_full(gpu_lib, 1, 130, 2, 128, causal, seed=8, scale=sc)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("descending", [False, True])
def test_bf16_running_max_moves(gpu_lib, d, causal, descending):
    """Scores that climb along the keys raise each row's running maximum many
    times (about 100 log2 units over the row), so every block takes the
    rescaling path; falling scores keep the first block's maximum throughout."""
    B, N, H = 1, 1000, 2
    span = 100.0 / (math.sqrt(d) * math.log2(math.e))
    x = inputs.make_qkv_ramp(B, N, H, d, span, seed=31 + d, descending=descending)
    sc = d ** -0.5
    print(f"\n[fwd bf16] ramp d={d} causal={causal} descending={descending}", flush=True)
    o, lse = run_bf16(gpu_lib, x, causal, scale=sc)
    check_parity(x, sc, causal, o=o, lse=lse, what=f"ramp d{d} causal={causal} descending={descending}")


def test_bf16_causal_row0_is_v0(gpu_lib):
    """Causal row 0 sees only key 0: O_0 equals V_0 bit for bit."""
    x = inputs.make_qkv(2, 300, 4, 128, torch.bfloat16, seed=11)
    o, lse = run_bf16(gpu_lib, x, True)
    assert torch.equal(o[:, 0].cpu(), x["v"][:, 0])
    ql, kl = inputs.to_f64(x["q"][:, 0]), inputs.to_f64(x["k"][:, 0])
    ref = (ql * kl).sum(-1) / math.sqrt(128)          # [B, H]
    assert np.abs(inputs.to_f64(lse[:, :, 0]) - ref).max() <= 1e-3


def test_bf16_deterministic(gpu_lib):
    x = inputs.make_qkv(2, 1000, 4, 128, torch.bfloat16, seed=12)
    o1, l1 = run_bf16(gpu_lib, x, True)
    o2, l2 = run_bf16(gpu_lib, x, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bf16_long_causal_n16384_every_head(gpu_lib):
    """B=1 H=32 N=16384 d=128 causal, the benchmark's long-context forward,
    in its launch configuration: O and LSE of every head against the oracle
    by the parity rule (the oracle and the rule's terms run over chunks of
    query rows, so no N x N array is formed); causal row 0 equals V_0."""
    w = workloads.LONG_CAUSAL
    print(f"\n[fwd bf16] {w.name}", flush=True)
    x = inputs.make_qkv(w.B, w.N, w.H, w.d, torch.bfloat16, seed=w.seed, gain=w.gain)
    o, lse = run_bf16(gpu_lib, x, w.causal)
    assert torch.equal(o[:, 0].cpu(), x["v"][:, 0])
    check_parity(x, w.scale, w.causal, o=o, lse=lse, what=w.name)


def test_f32_single_head(gpu_lib):
    """fp32 path, B=1 H=1 N=1024 d=64, K/V blocks of 256: max-abs <= 1e-5 on O and LSE."""
    w = workloads.SINGLE_HEAD_F32
    print(f"\n[fwd f32] {w.name}", flush=True)
    x = inputs.make_qkv(w.B, w.N, w.H, w.d, torch.float32, seed=w.seed)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = gpu_lib.forward_f32(q, k, v, causal=False)
    torch.cuda.synchronize()
    ro, rl = oracle.forward(*(inputs.to_f64(x[n]) for n in ("q", "k", "v")), w.scale, False)
    assert_f32_close(inputs.to_f64(o), ro, "O")
    assert_f32_close(inputs.to_f64(lse), rl, "LSE")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 5, 129, 300, 513])
def test_f32_small_shapes(gpu_lib, N, d, causal):
    print(f"\n[fwd f32] N={N} d={d} causal={causal}", flush=True)
    x = inputs.make_qkv(2, N, 2, d, torch.float32, seed=200 + N)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = gpu_lib.forward_f32(q, k, v, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.forward(*(inputs.to_f64(x[n]) for n in ("q", "k", "v")), d ** -0.5, causal)
    assert_f32_close(inputs.to_f64(o), ro, "O")
    assert_f32_close(inputs.to_f64(lse), rl, "LSE")
