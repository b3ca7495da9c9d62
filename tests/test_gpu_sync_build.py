"""Synchronisation check: libfa_sync.so is the same kernels built with
-DFA_DEBUG_SYNC, where every wave waits for all of its memory operations and
meets the others at a barrier at each K/V block or query step and before each
refill of an LDS ring stage.  Nothing overlaps there, so a read that the normal
build's waits and barriers let race ahead of its data (or a load that
overwrote a stage still being read) would give different values.  Every
output must equal the normal build's bit for bit: forward, backward (both
kernels and the three-step form), grouped-query attention, sliding windows,
a long causal shape whose launch order alternates the sweeps, and the FP8
forward."""

import pytest
import torch

from exact_io_aware_55_amd import binding, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def sync_lib(gpu_lib):
    return binding.open_library(binding.SYNC_LIB_PATH)


def both(monkeypatch, sync_lib, fn):
    """fn() with the normal library, then with the synchronisation check build."""
    normal = fn()
    torch.cuda.synchronize()
    with monkeypatch.context() as m:
        m.setattr(binding, "_lib", sync_lib)
        checked = fn()
        torch.cuda.synchronize()
    return normal, checked


def assert_bitwise(normal, checked, what):
    for i, (a, b) in enumerate(zip(normal, checked)):
        assert torch.equal(a, b), f"{what}: output {i} differs from the synchronisation check build"


def fwd_bwd(x, causal, window=None, three_step=False):
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))

    def run():
        o, lse = binding.forward(q, k, v, causal=causal, window=window)
        if three_step:
            grads, _ = binding.backward_steps(q, k, v, o, do, lse, causal=causal, preprocess=True)
        else:
            grads = binding.backward(q, k, v, o, do, lse, causal=causal, window=window)
        return (o, lse, *grads)
    return run


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_shapes_bitwise(monkeypatch, sync_lib, d, causal):
    print(f"\n[sync] B2 H4 N1000 d{d} causal={causal}", flush=True)
    x = inputs.make_qkv(2, 1000, 4, d, torch.bfloat16, seed=51 + d, with_do=True)
    assert_bitwise(*both(monkeypatch, sync_lib, fwd_bwd(x, causal)), f"d{d} causal={causal}")


def test_three_step_backward_bitwise(monkeypatch, sync_lib):
    print("\n[sync] three-step backward B1 H4 N777 d128 causal", flush=True)
    x = inputs.make_qkv(1, 777, 4, 128, torch.bfloat16, seed=52, with_do=True)
    assert_bitwise(*both(monkeypatch, sync_lib, fwd_bwd(x, True, three_step=True)), "three-step")


@pytest.mark.parametrize("d", [64, 128])
def test_long_causal_alternating_sweeps_bitwise(monkeypatch, sync_lib, d):
    """N d 4 bytes >= 4 MiB: the launch order reverses every other generation."""
    N = 16384 if d == 64 else 8192
    print(f"\n[sync] B1 H8 N{N} d{d} causal", flush=True)
    x = inputs.make_qkv(1, N, 8, d, torch.bfloat16, seed=53, with_do=True)
    assert_bitwise(*both(monkeypatch, sync_lib, fwd_bwd(x, True)), f"N{N} d{d}")


def test_gqa_bitwise(monkeypatch, sync_lib):
    print("\n[sync] GQA B1 H8 Hkv2 N900 d128 causal", flush=True)
    x = inputs.make_qkv(1, 900, 8, 128, torch.bfloat16, seed=54, with_do=True, H_kv=2)
    assert_bitwise(*both(monkeypatch, sync_lib, fwd_bwd(x, True)), "gqa")


def test_window_bitwise(monkeypatch, sync_lib):
    print("\n[sync] window 300 B1 H4 N2000 d64", flush=True)
    x = inputs.make_qkv(1, 2000, 4, 64, torch.bfloat16, seed=55, with_do=True)
    assert_bitwise(*both(monkeypatch, sync_lib, fwd_bwd(x, True, window=300)), "window")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_bitwise(monkeypatch, sync_lib, causal):
    print(f"\n[sync] fp8 B2 H4 N1000 d128 causal={causal}", flush=True)
    x = inputs.make_qkv_fp8(2, 1000, 4, 128, seed=56)
    args = [x[n].to(DEV) for n in ("q8", "k8", "v8", "q_descale", "k_descale", "v_descale")]
    normal, checked = both(monkeypatch, sync_lib, lambda: binding.forward_fp8(*args, causal=causal))
    assert_bitwise(normal, checked, f"fp8 causal={causal}")
