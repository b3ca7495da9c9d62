"""GPU parity of the FP8 forward (fa_fwd_fp8) against the fp64 oracle on the
decoded inputs, through the C ABI.

Tolerance (derived from the kernel's arithmetic, see ``parity.fp8_fwd_error_bound``):
every element of O within the first-order bound of rounding P to E4M3 plus
the bf16 output rounding; relative L2 of each head within twice the error
expected from independent E4M3 roundings; LSE (from unrounded P) within
1e-3 like the bf16 path.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_55_amd import inputs
from parity import (assert_lse_close, assert_within_bound, fp8_fwd_error_bound, fp8_fwd_rel_l2_limit,
                    rel_l2)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("q8", "k8", "v8", "q_descale", "k_descale", "v_descale")


def run(lib, x, causal, window=None, scale=None):
    args = [x[n].to(DEV) for n in NAMES]
    o, lse = lib.forward_fp8(*args, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def decoded(x):
    return [oracle.dequantize(x[n + "8"].numpy(), x[n + "_descale"].numpy()) for n in "qkv"]


def check_heads(o, lse, x, scale, causal, window, what, heads=None):
    q, k, v = decoded(x)
    B, N, H, d = q.shape
    G = H // k.shape[2]
    got_o, got_l = inputs.to_f64(o), inputs.to_f64(lse)
    for b, h in heads or [(b, h) for b in range(B) for h in range(H)]:
        args = (q[b, :, h], k[b, :, h // G], v[b, :, h // G], scale, causal)
        ro, rl = oracle.head_forward(*args, window=window)
        tag = f"{what} head {(b, h)}"
        assert np.all(np.isfinite(got_o[b, :, h])), f"{tag}: non-finite output"
        assert_within_bound(got_o[b, :, h], ro, fp8_fwd_error_bound(*args, window), tag, slack=1.0)
        lim = fp8_fwd_rel_l2_limit(*args, window)
        rl2 = rel_l2(got_o[b, :, h], ro)
        assert rl2 <= lim, f"{tag}: rel_l2 {rl2:.3e} > {lim:.3e}"
        assert_lse_close(got_l[b, h], rl, tag)


# (B, N, H, H_kv, d, causal, window): several tiles and ragged tails, both
# head sizes, grouped K/V heads, sliding windows, a single row
SHAPES = [
    (2, 300, 4, 4, 128, False, None),
    (1, 129, 4, 2, 64, True, None),
    (2, 1000, 4, 4, 128, True, None),
    (1, 65, 2, 2, 64, False, None),
    (1, 513, 4, 4, 128, True, 100),
    (1, 700, 4, 1, 64, True, 129),
    (1, 1, 2, 2, 128, False, None),
    (1, 2048, 2, 2, 128, False, None),
    # 24 heads split evenly over the 8 XCDs (3 each): the causal grid takes
    # them in pairs, the last group a single head
    (1, 1024, 24, 24, 128, True, None),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_N{}_H{}_Hkv{}_d{}_c{}_w{}".format(*s))
def test_fp8_forward(gpu_lib, shape):
    B, N, H, Hkv, d, causal, window = shape
    print(f"\n[fp8 fwd] {shape}", flush=True)
    x = inputs.make_qkv_fp8(B, N, H, d, seed=700 + N, H_kv=Hkv)
    o, lse = run(gpu_lib, x, causal, window)
    check_heads(o, lse, x, d ** -0.5, causal, window, str(shape))


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.3])
def test_fp8_forward_scales(gpu_lib, scale):
    """Zero scale (the mean of V), a negative scale (row minima), a large one."""
    x = inputs.make_qkv_fp8(1, 300, 2, 128, seed=31)
    o, lse = run(gpu_lib, x, True, scale=scale)
    check_heads(o, lse, x, scale, True, None, f"scale={scale}")


def test_fp8_forward_deterministic(gpu_lib):
    x = inputs.make_qkv_fp8(2, 777, 4, 128, seed=32, H_kv=2)
    o1, l1 = run(gpu_lib, x, True)
    o2, l2 = run(gpu_lib, x, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("w", [300, 2 ** 31 - 1])
def test_fp8_window_at_least_n_is_causal_bitwise(gpu_lib, w):
    """A window of N or more (here N and INT_MAX) hides no key: the result is
    plain causal attention bit for bit."""
    x = inputs.make_qkv_fp8(1, 300, 4, 128, seed=38, H_kv=2)
    o1, l1 = run(gpu_lib, x, True, window=w)
    o2, l2 = run(gpu_lib, x, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_bad_descale_gives_nan_rows_of_that_head_only(gpu_lib):
    x = inputs.make_qkv_fp8(1, 200, 4, 64, seed=33, H_kv=2)
    x["k_descale"][0, 1] = 0.0                     # K/V head 1 serves query heads 2 and 3
    o, lse = run(gpu_lib, x, False)
    on = inputs.to_f64(o)
    assert np.all(np.isnan(on[0, :, 2:])) and np.all(np.isnan(inputs.to_f64(lse)[0, 2:]))
    x["k_descale"][0, 1] = 1.0
    check_heads(o, lse, x, 64 ** -0.5, False, None, "healthy heads", heads=[(0, 0), (0, 1)])


@pytest.fixture(scope="module")
def fp8_c2_run(gpu_lib):
    """The FP8 forward at the forward benchmark shape (B=4 H=32 N=4096 d=128,
    non-causal), in the launch configuration the benchmark times."""
    x = inputs.make_qkv_fp8(4, 4096, 32, 128, seed=38)
    o, lse = run(gpu_lib, x, False)
    return x, o.cpu(), lse.cpu()


@pytest.mark.parametrize("b", [0, 1, 2, 3])
def test_fp8_forward_full_size_every_head(fp8_c2_run, b):
    """Every head of batch entry b at the benchmark shape: each element of O
    within the E4M3 bound, the head's relative L2 and LSE."""
    x, o, lse = fp8_c2_run
    print(f"\n[fp8 fwd] B4 N4096 H32 d128 b={b}", flush=True)
    check_heads(o, lse, x, 128 ** -0.5, False, None, f"b={b}", heads=[(b, h) for h in range(32)])


def test_fp8_forward_full_size_sampled(gpu_lib):
    """B=4 H=32 N=4096 d=128 non-causal (the forward benchmark shape), in the
    launch configuration the benchmark times: sampled rows against the
    oracle's rows, each within the element-wise bound."""
    B, N, H, d = 4, 4096, 32, 128
    print(f"\n[fp8 fwd] full size B{B} N{N} H{H} d{d}", flush=True)
    x = inputs.make_qkv_fp8(B, N, H, d, seed=34)
    o, lse = run(gpu_lib, x, False)
    q, k, v = decoded(x)
    got_o, got_l = inputs.to_f64(o), inputs.to_f64(lse)
    picks = inputs.pick_rows(B, H, N, 48, seed=35)
    for b, h, i in picks:
        args = (q[b, :, h], k[b, :, h], v[b, :, h], d ** -0.5, False)
        ro, rl = oracle.head_forward(*args, rows=[i])
        bd = fp8_fwd_error_bound(*args, rows=[i])
        assert_within_bound(got_o[b, i, h][None], ro, bd, f"row {(b, h, i)}", slack=1.0)
        assert abs(got_l[b, h, i] - rl[0]) <= 1e-3


def test_fp8_forward_long_causal_sampled(gpu_lib):
    """B=1 H=32 N=16384 d=128 causal (the second FP8 benchmark shape): sampled
    rows against the oracle's rows, each within the element-wise bound."""
    B, N, H, d = 1, 16384, 32, 128
    print(f"\n[fp8 fwd] long causal B{B} N{N} H{H} d{d}", flush=True)
    x = inputs.make_qkv_fp8(B, N, H, d, seed=36)
    o, lse = run(gpu_lib, x, True)
    q, k, v = decoded(x)
    got_o, got_l = inputs.to_f64(o), inputs.to_f64(lse)
    for b, h, i in inputs.pick_rows(B, H, N, 24, seed=37):
        args = (q[b, :, h], k[b, :, h], v[b, :, h], d ** -0.5, True)
        ro, rl = oracle.head_forward(*args, rows=[i])
        bd = fp8_fwd_error_bound(*args, rows=[i])
        assert_within_bound(got_o[b, i, h][None], ro, bd, f"row {(b, h, i)}", slack=1.0)
        assert abs(got_l[b, h, i] - rl[0]) <= 1e-3
