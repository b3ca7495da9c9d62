"""GPU parity of grouped-query attention (fa_fwd_gqa, fa_bwd_gqa) against the
fp64 oracle, through the C ABI: K and V have H_kv heads, each shared by
H / H_kv query heads (explainer page "Flash Attention", section "Varianten
und Erweiterungen", subsection "Grouped Query Attention")."""

import pytest
import torch

from exact_io_aware_55_amd import inputs
from parity import check_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def make(B, N, H, Hkv, d, seed):
    return inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=seed, with_do=True, H_kv=Hkv)


def fwd(lib, x, causal):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = lib.forward(q, k, v, causal=causal)
    torch.cuda.synchronize()
    return o, lse


# (B, N, H, H_kv, d): GQA groups of 2, 3 and 8, multi-query (H_kv = 1), ragged N
SHAPES = [(2, 300, 4, 2, 128), (1, 129, 6, 3, 64), (2, 1000, 8, 1, 128), (1, 65, 8, 4, 64),
          (1, 513, 16, 2, 128)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_N{}_H{}_Hkv{}_d{}".format(*s))
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_forward(gpu_lib, shape, causal):
    B, N, H, Hkv, d = shape
    print(f"\n[gqa fwd] {shape} causal={causal}", flush=True)
    x = make(B, N, H, Hkv, d, seed=500 + N)
    o, lse = fwd(gpu_lib, x, causal)
    check_parity(x, d ** -0.5, causal, o=o, lse=lse, what=f"{shape} causal={causal}")


def test_gqa_forward_matches_mha_on_repeated_kv(gpu_lib):
    """The grouped kernel on K/V equals the multi-head kernel on K/V heads
    copied to their query heads, bit for bit (same tiles, same order)."""
    B, N, H, Hkv, d = 2, 700, 8, 2, 128
    x = make(B, N, H, Hkv, d, seed=77)
    for causal in (False, True):
        o, lse = fwd(gpu_lib, x, causal)
        rep = {"q": x["q"], "k": x["k"].repeat_interleave(H // Hkv, dim=2).contiguous(),
               "v": x["v"].repeat_interleave(H // Hkv, dim=2).contiguous()}
        o2, lse2 = fwd(gpu_lib, rep, causal)
        assert torch.equal(o, o2) and torch.equal(lse, lse2)


def check_bwd(lib, B, N, H, Hkv, d, causal, seed, groups=None):
    """dQ of every query head and the group-summed dK, dV of each listed K/V
    head (default all) by the parity rule."""
    x = make(B, N, H, Hkv, d, seed)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = lib.forward(q, k, v, causal=causal)
    dq, dk, dv = lib.backward(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    check_parity(x, d ** -0.5, causal, o=o, lse=lse, grads=(dq, dk, dv), groups=groups,
                 what=f"B{B} N{N} H{H} Hkv{Hkv} d{d} causal={causal}")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_N{}_H{}_Hkv{}_d{}".format(*s))
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward(gpu_lib, shape, causal):
    B, N, H, Hkv, d = shape
    print(f"\n[gqa bwd] {shape} causal={causal}", flush=True)
    check_bwd(gpu_lib, B, N, H, Hkv, d, causal, seed=600 + N)


def test_gqa_backward_full_size_group(gpu_lib):
    """H = 64 query heads over 8 K/V heads (the page's Llama 2 70B ratio),
    N = 2048, d = 128: one whole group checked against the oracle."""
    print("\n[gqa bwd] B1 N2048 H64 Hkv8 d128 causal", flush=True)
    check_bwd(gpu_lib, 1, 2048, 64, 8, 128, True, seed=901, groups=[(0, 5)])


def test_gqa_backward_long_causal_alternating_sweeps(gpu_lib):
    """N = 8192, d = 128 causal: a head's K/V exceed one XCD's L2, so the
    launch order reverses every other generation; the key-block kernel then
    walks the query blocks of all four heads of a group in reverse order.
    One K/V group (dK, dV summed over its heads) by the parity rule."""
    print("\n[gqa bwd] B1 N8192 H8 Hkv2 d128 causal", flush=True)
    check_bwd(gpu_lib, 1, 8192, 8, 2, 128, True, seed=902, groups=[(0, 1)])


def test_gqa_bad_group_count_is_rejected(gpu_lib):
    x = make(1, 64, 6, 3, 64, seed=1)
    q = x["q"].to(DEV)
    k = x["q"].to(DEV)[:, :, :4].contiguous()     # 4 K/V heads do not divide 6
    with pytest.raises(ValueError):
        gpu_lib.forward(q, k, k, causal=False)
