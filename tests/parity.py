"""Comparison helpers for GPU-vs-oracle parity (tolerances from the method's
accuracy targets: fp32 path max-abs <= 1e-5; bf16 path O, dQ, dK, dV max-abs
<= 2e-2 and relative L2 <= 5e-3; LSE max-abs <= 1e-3)."""

import numpy as np

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


def max_abs(got, ref):
    return float(np.abs(np.asarray(got, np.float64) - ref).max()) if np.size(ref) else 0.0


def rel_l2(got, ref):
    num = np.linalg.norm((np.asarray(got, np.float64) - ref).ravel())
    den = np.linalg.norm(np.asarray(ref, np.float64).ravel())
    return float(num / den) if den > 0 else float(num)


def assert_bf16_close(got, ref, what=""):
    ma, rl = max_abs(got, ref), rel_l2(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert ma <= BF16_MAX_ABS and rl <= BF16_REL_L2, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}"
    return ma, rl


def assert_lse_close(got, ref, what=""):
    ma = max_abs(got, ref)
    assert ma <= LSE_MAX_ABS, f"{what}: lse max_abs={ma:.3e}"
    return ma


def assert_f32_close(got, ref, what=""):
    ma = max_abs(got, ref)
    assert ma <= F32_MAX_ABS, f"{what}: max_abs={ma:.3e}"
    return ma
