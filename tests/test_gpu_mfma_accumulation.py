"""GPU measurement of the matrix cores' accumulation error, which the FP8
forward's error bound (tests/parity.py, FP8_MFMA_ACC) and the bf16 parity
rule's fp32 terms rely on.

fa_probe_mfma multiplies 32 x 32 tiles on the same MFMA instructions the
kernels use (v_mfma_f32_32x32x64_f8f6f4 for E4M3 codes, v_mfma_f32_32x32x16_bf16
for bf16), chaining k / 64 or k / 16 of them in one fp32 accumulator.  Every
product of two E4M3 or two bf16 values is exact in fp64, so the fp64 sum is
the exact result; the error of each output element is measured relative to
the sum of the absolute values of its products, the quantity the bounds
scale with.  The inputs cover random codes over the whole finite range,
sums with heavy cancellation and products of very different sizes."""

import math

import numpy as np
import pytest
import torch

from parity import FP8_MFMA_ACC

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16_MFMA_ACC = 2.0 ** -16     # allowance for the bf16 MFMA accumulation (relative to sum |a b|)


def e4m3_codes(g, shape):
    """Random E4M3 codes: every finite code equally likely (0x7f and 0xff are NaN)."""
    c = g.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)


def decode_e4m3(codes):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def cases_e4m3(k, seed):
    g = np.random.default_rng(seed)
    t = 128
    a, b = e4m3_codes(g, (t, 32, k)), e4m3_codes(g, (t, 32, k))
    # heavy cancellation: the second half of each row repeats the first with
    # the sign flipped (0x80), plus a few untouched entries
    a2, b2 = a.copy(), b.copy()
    h = k // 2
    a2[:, :, h:] = a2[:, :, :h] ^ 0x80
    b2[:, :, h:] = b2[:, :, :h]
    a2[:, :, ::17] = e4m3_codes(g, a2[:, :, ::17].shape)
    # products of very different sizes: one large pair per row, the rest tiny
    a3 = g.integers(0x00, 0x10, size=(t, 32, k), dtype=np.uint8) | (g.integers(0, 2, (t, 32, k)) << 7).astype(np.uint8)
    b3 = g.integers(0x00, 0x10, size=(t, 32, k), dtype=np.uint8)
    a3[:, :, 5] = 0x7E
    b3[:, :, 5] = 0x7E
    return [("random", a, b), ("cancelling", a2, b2), ("mixed sizes", a3, b3)]


def relative_error(got, a, b):
    exact = np.einsum("tij,tcj->tic", a, b)
    scale = np.einsum("tij,tcj->tic", np.abs(a), np.abs(b))
    err = np.abs(got - exact)
    return float(np.max(np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), err)))


@pytest.mark.parametrize("k", [128, 1024])
def test_fp8_mfma_accumulation_within_allowance(gpu_lib, k):
    """E4M3 MFMA: every output within FP8_MFMA_ACC (2^-11) of sum |a b|;
    k = 128 is the score product at d = 128, k = 1024 a P V chain over 1024
    keys."""
    worst = 0.0
    for name, ca, cb in cases_e4m3(k, seed=k):
        c = gpu_lib.probe_mfma(torch.from_numpy(ca).to(DEV), torch.from_numpy(cb).to(DEV), fp8=True)
        torch.cuda.synchronize()
        rel = relative_error(c.double().cpu().numpy(), decode_e4m3(ca), decode_e4m3(cb))
        print(f"\n[fp8 mfma] k={k} {name}: max error / sum|ab| = 2^{math.log2(max(rel, 1e-300)):.1f}", flush=True)
        worst = max(worst, rel)
    assert worst <= FP8_MFMA_ACC


@pytest.mark.parametrize("k", [128, 1024])
def test_bf16_mfma_accumulation_within_allowance(gpu_lib, k):
    """bf16 MFMA: every output within 2^-16 of sum |a b| (the bf16 parity
    rule's vector terms are per-rounding u = 2^-8, far above this)."""
    g = np.random.default_rng(1000 + k)
    t = 128
    a = torch.from_numpy(g.standard_normal((t, 32, k)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy(g.standard_normal((t, 32, k)).astype(np.float32)).to(torch.bfloat16)
    b_c = b.clone()
    b_c[:, :, k // 2:] = b_c[:, :, :k // 2]
    a_c = a.clone()
    a_c[:, :, k // 2:] = -a_c[:, :, :k // 2]
    worst = 0.0
    for name, x, y in (("random", a, b), ("cancelling", a_c, b_c)):
        c = gpu_lib.probe_mfma(x.to(DEV), y.to(DEV), fp8=False)
        torch.cuda.synchronize()
        rel = relative_error(c.double().cpu().numpy(), x.double().numpy(), y.double().numpy())
        print(f"\n[bf16 mfma] k={k} {name}: max error / sum|ab| = 2^{math.log2(max(rel, 1e-300)):.1f}", flush=True)
        worst = max(worst, rel)
    assert worst <= BF16_MFMA_ACC


def test_probe_is_the_exact_product_on_small_integers(gpu_lib):
    """Small integers multiply and add exactly in both formats: the probe's
    tile layout (rows, columns, contraction slots) must reproduce A B^T bit
    for bit.  A transposed tile or a dropped chunk would not."""
    g = np.random.default_rng(7)
    a = g.integers(-3, 4, size=(8, 32, 128)).astype(np.float32)
    b = g.integers(-3, 4, size=(8, 32, 128)).astype(np.float32)
    exact = np.einsum("tij,tcj->tic", a, b)
    c = gpu_lib.probe_mfma(torch.from_numpy(a).to(torch.bfloat16).to(DEV),
                           torch.from_numpy(b).to(torch.bfloat16).to(DEV), fp8=False)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), exact)
    codes_a = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8)
    codes_b = torch.from_numpy(b).to(torch.float8_e4m3fn).view(torch.uint8)
    c8 = gpu_lib.probe_mfma(codes_a.to(DEV), codes_b.to(DEV), fp8=True)
    torch.cuda.synchronize()
    assert np.array_equal(c8.cpu().numpy(), exact)
