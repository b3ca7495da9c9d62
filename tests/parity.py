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


def assert_bf16_close(got, ref, what="", terms=1):
    """Fixed bf16 tolerances.  ``terms``: the output is a sum of that many
    per-head gradients (a K/V head shared by a group of query heads); the
    max-abs bound is per head, so it applies to the group mean (the sum's
    bound scales by ``terms``), and the scale-free relative L2 is unchanged."""
    ma, rl = max_abs(got, ref), rel_l2(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert ma <= BF16_MAX_ABS * terms and rl <= BF16_REL_L2, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}"
    return ma, rl


def assert_lse_close(got, ref, what=""):
    ma = max_abs(got, ref)
    assert ma <= LSE_MAX_ABS, f"{what}: lse max_abs={ma:.3e}"
    return ma


def assert_f32_close(got, ref, what=""):
    ma = max_abs(got, ref)
    assert ma <= F32_MAX_ABS, f"{what}: max_abs={ma:.3e}"
    return ma


# --------------------------------------------------------------------------
# Element-wise a-priori error bound of the bf16 backward arithmetic.
#
# The bf16 path rounds (round to nearest even, unit roundoff u = 2^-8) the
# forward's O, the probabilities P before dV = P^T dO, dS before dK and dQ,
# and each output once; everything else accumulates in fp32.  First-order
# propagation of those roundings gives, per element:
#   |dO_err| row statistic:  dD_i  <= sum_k |dO_ik| (u|O_ik| + u (P|V|)_ik)
#   dS error:                edS_ij <= P_ij dD_i + u |dS_ij|
#   dV: u (P^T|dO|) + u|dV|
#   dK: |scale| (edS^T |Q|) + u|dK|
#   dQ: |scale| (edS |K|) + u|dQ|
# plus an fp32 accumulation allowance.  A correct kernel stays inside this
# bound at any size and scale, including degenerate shapes where the fixed
# max-abs / relative-L2 tolerances are tighter than the bf16 arithmetic allows.
# --------------------------------------------------------------------------
U_BF16 = 2.0 ** -8
F32_ALLOW = 1e-5


def bwd_error_bounds(q, k, v, do, scale, causal, window=None):
    """Return (bound_dQ, bound_dK, bound_dV) for one head (fp64 inputs)."""
    import oracle

    p, _, _ = oracle.head_probabilities(q, k, scale, causal, window=window)
    o = p @ v
    dp = do @ v.T
    delta = (p * dp).sum(1)
    ds = p * (dp - delta[:, None])
    dq, dk, dv = oracle.head_backward(q, k, v, do, scale, causal, window)
    u = U_BF16
    o_err = u * np.abs(o) + u * (p @ np.abs(v))
    d_err = (np.abs(do) * o_err).sum(1)
    eds = p * d_err[:, None] + u * np.abs(ds)
    s = abs(scale)
    b_dv = u * (p.T @ np.abs(do)) + u * np.abs(dv) + F32_ALLOW * (p.T @ np.abs(do))
    b_dk = s * (eds.T @ np.abs(q)) + u * np.abs(dk) + F32_ALLOW * s * (np.abs(ds).T @ np.abs(q))
    b_dq = s * (eds @ np.abs(k)) + u * np.abs(dq) + F32_ALLOW * s * (np.abs(ds) @ np.abs(k))
    return b_dq, b_dk, b_dv


def assert_within_bound(got, ref, bound, what="", slack=1.25):
    err = np.abs(np.asarray(got, np.float64) - ref)
    lim = slack * bound + 1e-6
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements outside the bf16 rounding bound; "
                           f"worst excess {float((err - lim).max()):.3e}")


# --------------------------------------------------------------------------
# Element-wise a-priori error bound of the FP8 forward.
#
# The oracle is attention of the decoded E4M3 inputs, so the inputs carry no
# error.  The kernel then rounds each probability p (in its own units, where
# p <= 2^8 because the running maximum lags the true one by at most 8 in
# log2 units) to E4M3 for the P V product: |p~ - p| <= 2^-4 p in the normal
# range and <= 2^-10 (half the subnormal spacing) below 2^-6.  The row sum l
# adds the unrounded fp32 p, and l >= L_i = sum_j exp(s_ij - max_j s_ij)
# whatever maximum was used.  So, per output element,
#   |O_err| <= 2^-4 (P|V|) + 2^-10 (sum_vis |V|) / L_i
# plus the score error of the fp8 matrix core (its accumulation was measured
# at about 2^-15 of sum |a b|; allowed here as 2^-12, which perturbs each p by
# a relative eta_i <= 2^-11 |scale| max_j (|q_i| . |k_j|)), the same allowance
# on the P V accumulation, the bf16 rounding of O (2^-8 |O|) and fp32 terms.
# --------------------------------------------------------------------------
U_E4M3 = 2.0 ** -4
SUB_E4M3 = 2.0 ** -10
FP8_MFMA_ACC = 2.0 ** -12


def fp8_fwd_error_bound(q, k, v, scale, causal, window=None, rows=None):
    """Element-wise bound on |O_gpu - O_oracle| for one head (fp64 decoded
    inputs); ``rows`` restricts it to those query rows."""
    import oracle

    p, m, _ = oracle.head_probabilities(q, k, scale, causal, rows=rows, window=window)
    if rows is not None:
        q = q[np.asarray(rows)]
    vis = p > 0
    s = scale * (q @ k.T)
    # L_i = sum_j exp(s_ij - max_j s_ij) over visible keys
    big_l = np.where(vis, np.exp(np.where(vis, s, 0.0) - m[:, None]), 0.0).sum(1)
    pv = p @ np.abs(v)
    o = np.abs(p @ v)
    eta = 2.0 ** -11 * abs(scale) * (np.abs(q) @ np.abs(k).T).max(1)
    return ((U_E4M3 + FP8_MFMA_ACC + 2.0 ** -16) * pv + SUB_E4M3 * (vis @ np.abs(v)) / big_l[:, None]
            + (U_BF16 + 2.0 ** -16) * o + eta[:, None] * (pv + o) + 1e-7)


def fp8_fwd_rel_l2_limit(q, k, v, scale, causal, window=None, factor=2.0):
    """Relative-L2 limit for the FP8 forward of one head: ``factor`` times the
    root-mean-square error expected from independent E4M3 roundings of P
    (relative error spread evenly over +-2^-4: standard deviation
    2^-4 / sqrt(3)), i.e. sqrt(sum_ij sigma^2 P_ij^2 |V_j|^2) / ||P V||."""
    import oracle

    p, _, _ = oracle.head_probabilities(q, k, scale, causal, window=window)
    sigma = U_E4M3 / np.sqrt(3.0)
    expected = sigma * np.sqrt(((p ** 2) @ (v ** 2)).sum())
    return factor * float(expected / np.linalg.norm(p @ v))
