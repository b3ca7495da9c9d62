"""Comparison helpers for GPU-vs-oracle parity (tolerances from the method's
accuracy targets: fp32 path max-abs <= 1e-5; bf16 path O, dQ, dK, dV max-abs
<= 2e-2 and relative L2 <= 5e-3; LSE max-abs <= 1e-3)."""

import concurrent.futures as cf
import os

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


def assert_lse_close(got, ref, what=""):
    ma = max_abs(got, ref)
    assert ma <= LSE_MAX_ABS, f"{what}: lse max_abs={ma:.3e}"
    return ma


def assert_f32_close(got, ref, what=""):
    ma = max_abs(got, ref)
    assert ma <= F32_MAX_ABS, f"{what}: max_abs={ma:.3e}"
    return ma


# --------------------------------------------------------------------------
# The bf16 parity rule.
#
# The method is exact up to rounding, and the contract puts two lines on the
# bf16 outputs O, dQ, dK and dV: max-abs error <= TAU = 2e-2 and relative L2
# error <= RHO = 5e-3.  The bf16 path itself rounds (unit roundoff
# u = 2^-8, round to nearest even): each probability P before P V and before
# dV = P^T dO, each dS before dK and dQ, the forward's O (which the backward
# reads to form D = rowsum(dO * O)), and every output once.  Those roundings
# alone can cross the fixed lines: an output of magnitude 8 or more has a
# half-spacing of 2^-5 > TAU, and a key that many queries attend to (causal
# key 0 collects sum_i P_i0 ~ ln N) gathers the rounding errors of all those
# probabilities.  So every test applies ONE rule, to every element and every
# (batch, head) of every bf16 output X with oracle value X*:
#
#   (R1) |X_e - X*_e| <= max(TAU, min(W_e, Z sigma_e)),            Z = 6
#   (R2) ||X - X*||_2  <= max(RHO ||X*||_2, KAPPA sqrt(sum_e sigma_e^2)),  KAPPA = 1.5
#
# W_e is the first-order worst case of those roundings at element e (every
# rounding error at its largest, all of one sign), a hard bound.  sigma_e is
# the standard deviation of the same error when every rounding is an
# independent relative error spread evenly over [-u, u] (variance u^2 / 3,
# an upper bound for round-to-nearest), with the error of D shared by all
# entries of its row.  An element sums many independent roundings, so its
# error stays within a few sigma long before it can reach W; Z = 6 takes the
# smaller of the two.  The fixed line is replaced only where that model says
# a correct kernel can cross it.  fp32 arithmetic enters through small
# relative terms: a d-term fp32 score (bounded through Cauchy-Schwarz), the
# exponent's subtraction and the exp2 instruction (eta), and 4 sqrt(n) 2^-24
# per n-term fp32 sum (a probabilistic bound; the worst case n 2^-24 would
# exceed u itself at large n), with standard deviation sqrt(n / 3) 2^-24.
# The bf16 matrix core accumulates to fp32 accuracy
# (tests/test_gpu_mfma_accumulation.py measures 2^-23.4 of sum |a b|).
# --------------------------------------------------------------------------
U_BF16 = 2.0 ** -8
TAU = BF16_MAX_ABS
RHO = BF16_REL_L2
Z_ELEM = 6.0
KAPPA = 1.5
SECOND_ORDER = 1.0 + 2.0 ** -6      # products of two roundings: u^2 / u = 2^-8 of the first-order terms
ROW_CHUNK = 1024                    # query rows per chunk (bounds memory at long N)
VAR_U = U_BF16 ** 2 / 3.0


def fp32_sum_rel(n):
    """Relative error allowance of an fp32 sum of n terms (times the sum of
    their absolute values): 4 sqrt(n) 2^-24."""
    return 4.0 * np.sqrt(np.maximum(n, 1)) * 2.0 ** -24


def fp32_sum_sd(n):
    """Standard deviation of the same error, relative to the sum of absolute
    values: sqrt(n / 3) 2^-24."""
    return np.sqrt(np.maximum(n, 1) / 3.0) * 2.0 ** -24


class Terms:
    """Propagated rounding terms of one output tensor, before the tensor's own
    bf16 rounding: the oracle value, the worst case W and the variance."""

    def __init__(self, exact, worst, var):
        self.exact, self.worst, self.var = exact, worst, var

    def __add__(self, other):            # gradients of one K/V head summed over its query heads
        return Terms(self.exact + other.exact, self.worst + other.worst, self.var + other.var)


def _row_eta(q, k, scale, d):
    """Relative error of each probability before any bf16 rounding: the fp32
    score (a d-term dot product, bounded by Cauchy-Schwarz through the row's
    |q| and the largest |k|), the subtraction of the row maximum or LSE from
    it, and the exp2 instruction.  Per query row."""
    smax = abs(scale) * np.linalg.norm(q, axis=1) * np.linalg.norm(k, axis=1).max()
    return 2.0 ** -24 * (d * smax + 2.0 * smax * np.log2(np.e) + 4.0)


def head_rounding_terms(q, k, v, scale, causal, window=None, do=None, rows=None):
    """Rounding terms of one head's bf16 outputs.

    Returns ({"O": Terms} and, with ``do``, also "dQ", "dK", "dV"; and the
    oracle's LSE).  The exact values come from the oracle's own functions
    (head_forward, head_backward); W and the variance follow the roundings
    of the bf16 path listed above, computed over chunks of query rows.
    ``rows`` (forward only) restricts everything to those query rows."""
    import oracle

    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    N, d = q.shape
    u = U_BF16
    s_ = abs(scale)
    back = do is not None
    assert rows is None or not back, "rows: forward only"
    all_rows = np.arange(N) if rows is None else np.asarray(rows)
    chunks = [all_rows[i:i + ROW_CHUNK] for i in range(0, len(all_rows), ROW_CHUNK)]
    eta = _row_eta(q, k, scale, d)
    o_ex = np.empty((N, v.shape[1]))
    lse_ex = np.empty(N)
    for rs in chunks:
        o_ex[rs], lse_ex[rs] = oracle.head_forward(q, k, v, scale, causal, rows=rs, window=window)
    av, v2 = np.abs(v), v * v
    w_o, var_o = np.empty_like(o_ex), np.empty_like(o_ex)
    if back:
        do = np.asarray(do, np.float64)
        dq_ex, dk_ex, dv_ex = oracle.head_backward(q, k, v, do, scale, causal, window)
        aq, ak, q2, k2 = np.abs(q), np.abs(k), q * q, k * k
        ado, do2 = np.abs(do), do * do
        zeta = fp32_sum_rel(d) * np.linalg.norm(do, axis=1) * np.linalg.norm(v, axis=1).max()
        w_dq, var_dq = np.empty_like(dq_ex), np.empty_like(dq_ex)
        w_dk, var_dk = np.zeros_like(dk_ex), np.zeros_like(dk_ex)
        w_dv, var_dv = np.zeros_like(dv_ex), np.zeros_like(dv_ex)
        ads_q = np.zeros_like(dk_ex)       # |dS|^T |Q|
        pt_do = np.zeros_like(dv_ex)       # P^T |dO|
        n_col = np.zeros(N)                # queries that see each key
    for ci, rows in enumerate(chunks):
        p, _, _ = oracle.head_probabilities(q, k, scale, causal, rows=rows, window=window)
        p2 = p * p
        n_vis = (p > 0).sum(1)
        e_r = eta[rows]
        pav = p @ av
        # forward: P rounded before P V (relative u, on top of eta), the row
        # sum l of the unrounded fp32 P (relative eta + fp32 sum, shared by
        # the row), the P V accumulation in fp32
        w_o[rows] = (u + 2.0 * e_r + 2.0 * fp32_sum_rel(n_vis))[:, None] * pav
        var_o[rows] = ((VAR_U + e_r ** 2 / 3.0)[:, None] * (p2 @ v2)
                       + ((e_r / np.sqrt(3.0) + fp32_sum_sd(n_vis))[:, None] * o_ex[rows]) ** 2
                       + (fp32_sum_sd(n_vis)[:, None] * pav) ** 2)
        if not back:
            continue
        # the recomputed P = exp2(S scale log2 e - LSE log2 e) also carries the
        # error of the forward's fp32 LSE (its row sum, and its own rounding)
        e_b = e_r + fp32_sum_rel(n_vis) + 2.0 ** -24 * (2.0 + np.abs(lse_ex[rows]))
        # the O the backward reads is the bf16 forward output
        o_r = o_ex[rows]
        wo_tot = SECOND_ORDER * w_o[rows] + u * np.abs(o_r)
        vo_tot = var_o[rows] + VAR_U * o_r * o_r
        # D_i = dO_i . O_i in fp32
        doo = (ado[rows] * np.abs(o_r)).sum(1)
        w_d = (ado[rows] * wo_tot).sum(1) + fp32_sum_rel(d) * doo
        var_d = (do2[rows] * vo_tot).sum(1) + (fp32_sum_sd(d) * doo) ** 2
        dp = do[rows] @ v.T
        delta = (do[rows] * o_r).sum(1)
        ds = p * (dp - delta[:, None])
        ads = np.abs(ds)
        # dS = P (dP - D): D's error (shared along the row), dP's fp32 error,
        # P's fp32 error, then dS rounded to bf16 before dK and dQ
        zr = zeta[rows][:, None]
        w_ds = p * (w_d[:, None] + zr) + (u + e_b)[:, None] * ads
        var_ds = (VAR_U + e_b ** 2 / 3.0)[:, None] * ds * ds + p2 * zr * zr / 48.0
        ads_k = ads @ ak
        # dQ_i = scale sum_j dS_ij K_j; D's error is common to the row, so it
        # scales (P K)_i as a whole
        w_dq[rows] = s_ * (w_ds @ ak) + s_ * fp32_sum_rel(n_vis)[:, None] * ads_k
        var_dq[rows] = scale * scale * (var_ds @ k2 + var_d[:, None] * (p @ k) ** 2
                                        + (fp32_sum_sd(n_vis)[:, None] * ads_k) ** 2)
        # dK_j = scale sum_i dS_ij Q_i; dV_j = sum_i bf16(P_ij) dO_i
        w_dk += s_ * (w_ds.T @ aq[rows])
        var_dk += scale * scale * (var_ds.T @ q2[rows] + (p2 * var_d[:, None]).T @ q2[rows])
        w_dv += ((u + e_b)[:, None] * p).T @ ado[rows]
        var_dv += ((VAR_U + e_b ** 2 / 3.0)[:, None] * p2).T @ do2[rows]
        ads_q += ads.T @ aq[rows]
        pt_do += p.T @ ado[rows]
        n_col += (p > 0).sum(0)
    sel = all_rows
    out = {"O": Terms(o_ex[sel], w_o[sel], var_o[sel])}
    if back:
        fk, fs = fp32_sum_rel(n_col)[:, None], fp32_sum_sd(n_col)[:, None]
        out["dQ"] = Terms(dq_ex, w_dq, var_dq)
        out["dK"] = Terms(dk_ex, w_dk + s_ * fk * ads_q, var_dk + (scale * fs * ads_q) ** 2)
        out["dV"] = Terms(dv_ex, w_dv + fk * pt_do, var_dv + (fs * pt_do) ** 2)
    return out, lse_ex[sel]


def rule_limits(t: Terms):
    """(element limits of R1, L2 limit of R2) for one output tensor."""
    worst = SECOND_ORDER * t.worst + U_BF16 * np.abs(t.exact) + 1e-7
    var = t.var + VAR_U * t.exact * t.exact
    elem = np.maximum(TAU, np.minimum(worst, Z_ELEM * np.sqrt(var) + 1e-7))
    l2 = max(RHO * float(np.linalg.norm(t.exact)), KAPPA * float(np.sqrt(var.sum())))
    return elem, l2


def check_bf16(got, t: Terms, what=""):
    """Apply the parity rule (R1, R2) to one output tensor of one head (or one
    K/V head's group sum).  Returns a dict of the observed errors."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    elem, l2_lim = rule_limits(t)
    err = np.abs(got - t.exact)
    bad = err > elem
    if bad.any():
        i = int(np.argmax((err - elem).ravel()))
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond max(2e-2, min(W, 6 sigma)); "
                             f"error {float(err.ravel()[i]):.3e} where the limit is {float(elem.ravel()[i]):.3e}")
    l2 = float(np.linalg.norm(err))
    ref = float(np.linalg.norm(t.exact))
    assert l2 <= l2_lim, f"{what}: L2 error {l2:.3e} > {l2_lim:.3e} (relative {l2 / max(ref, 1e-300):.3e})"
    return {"max_abs": float(err.max()) if err.size else 0.0, "rel_l2": l2 / ref if ref > 0 else l2,
            "loosened_elems": int((elem > TAU).sum()), "loosened_l2": bool(l2_lim > RHO * ref)}


def _workers():
    """Threads for the per-head checks: the host cores available, at most 16
    (numpy releases the GIL in its array loops; BLAS runs one thread each)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _host(t):
    """A tensor's values as a host array (bf16 and fp32 widen exactly)."""
    if t is None:
        return None
    if hasattr(t, "detach"):
        return t.detach().to("cpu").float().numpy()
    return np.asarray(t)


def check_parity(x, scale, causal, o=None, lse=None, grads=None, window=None, groups=None, what=""):
    """The parity rule on every listed head.

    x: dict of host tensors 'q' [B,N,H,d], 'k', 'v' [B,N,H_kv,d] (and 'do'
    when ``grads`` is given), exactly the inputs the kernels received.
    o, lse: the forward's outputs (or None); grads: (dQ, dK, dV) or None.
    groups: (b, hk) K/V heads whose query heads are checked (default: all);
    dK and dV of a K/V head are checked against the group sum.  The heads
    run on a thread pool.  Returns a summary dict of the observed errors."""
    q, k, v = (_host(x[n]) for n in ("q", "k", "v"))
    do = _host(x["do"]) if grads is not None else None
    B, N, H, _ = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    og, lg = _host(o), _host(lse)
    gq, gk, gv = (_host(g) for g in grads) if grads is not None else (None, None, None)
    todo = groups if groups is not None else [(b, hk) for b in range(B) for hk in range(Hkv)]
    f64 = lambda a: np.asarray(a, np.float64)

    def one(bk):
        b, hk = bk
        kh, vh = f64(k[b, :, hk]), f64(v[b, :, hk])
        reps, tk, tv = [], None, None
        for h in range(hk * G, hk * G + G):
            tag = f"{what} head {(b, h)}"
            t, lse_ex = head_rounding_terms(f64(q[b, :, h]), kh, vh, scale, causal, window,
                                            None if do is None else f64(do[b, :, h]))
            if og is not None:
                reps.append(("O", check_bf16(og[b, :, h], t["O"], f"{tag} O")))
            if lg is not None:
                assert_lse_close(lg[b, h], lse_ex, tag)
            if gq is not None:
                reps.append(("dQ", check_bf16(gq[b, :, h], t["dQ"], f"{tag} dQ")))
                tk = t["dK"] if tk is None else tk + t["dK"]
                tv = t["dV"] if tv is None else tv + t["dV"]
        if gq is not None:
            reps.append(("dK", check_bf16(gk[b, :, hk], tk, f"{what} K/V head {(b, hk)} dK")))
            reps.append(("dV", check_bf16(gv[b, :, hk], tv, f"{what} K/V head {(b, hk)} dV")))
        return reps

    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(_workers()) as ex:
            results = list(ex.map(one, todo))
    summary = {}
    for reps in results:
        for name, r in reps:
            s_ = summary.setdefault(name, {"max_abs": 0.0, "rel_l2": 0.0, "loosened_elems": 0,
                                           "loosened_l2": 0, "tensors": 0})
            s_["max_abs"] = max(s_["max_abs"], r["max_abs"])
            s_["rel_l2"] = max(s_["rel_l2"], r["rel_l2"])
            s_["loosened_elems"] += r["loosened_elems"]
            s_["loosened_l2"] += int(r["loosened_l2"])
            s_["tensors"] += 1
    line = f"[parity] {what}: " + "; ".join(
        f"{n} max_abs {v['max_abs']:.2e} rel_l2 {v['rel_l2']:.2e} loosened {v['loosened_elems']} elems, "
        f"{v['loosened_l2']}/{v['tensors']} L2" for n, v in summary.items())
    print(line, flush=True)
    log = os.environ.get("FA_PARITY_LOG")
    if log:                              # a record of the observed errors per check
        with open(log, "a") as fh:
            fh.write(line + "\n")
    return summary


def check_rows_forward(o_rows, lse_rows, x, scale, causal, picks, window=None, what=""):
    """The parity rule on sampled forward rows (b, h, i): each row's O by the
    rule (R1 per element; R2 over the sampled rows of a head) and its LSE
    within 1e-3.  o_rows [len(picks), d], lse_rows [len(picks)]."""
    q, k, v = (_host(x[n]) for n in ("q", "k", "v"))
    H, Hkv = q.shape[2], k.shape[2]
    G = H // Hkv
    by_head = {}
    for n, (b, h, i) in enumerate(picks):
        by_head.setdefault((b, h), []).append((i, n))
    f64 = lambda a: np.asarray(a, np.float64)
    o_rows, lse_rows = np.asarray(o_rows, np.float64), np.asarray(lse_rows, np.float64)
    for (b, h), lst in by_head.items():
        rows = [i for i, _ in lst]
        idx = [n for _, n in lst]
        t, lse_ex = head_rounding_terms(f64(q[b, :, h]), f64(k[b, :, h // G]), f64(v[b, :, h // G]), scale,
                                        causal, window, rows=rows)
        check_bf16(o_rows[idx], t["O"], f"{what} head {(b, h)} rows")
        assert_lse_close(lse_rows[idx], lse_ex, f"{what} head {(b, h)} rows")


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
# plus the score error of the fp8 matrix core, the same allowance on the P V
# accumulation, the bf16 rounding of O (2^-8 |O|) and fp32 terms.  The E4M3
# matrix core does not accumulate exactly in fp32:
# tests/test_gpu_mfma_accumulation.py multiplies tiles on it
# (v_mfma_f32_32x32x64_f8f6f4, the kernel's instruction) and measures up to
# 2^-12.6 of sum |a b| for a 128-long contraction of random codes over the
# whole E4M3 range (2^-14.6 at 1024; the bf16 MFMA measures 2^-23.4, fp32
# exact), and holds every output to FP8_MFMA_ACC = 2^-11.  A score error of
# FP8_MFMA_ACC sum |q||k| moves each p by a relative
# eta_i <= 2 FP8_MFMA_ACC |scale| max_j (|q_i| . |k_j|) (the factor 2 covers
# the exponential's second order).
# --------------------------------------------------------------------------
def assert_within_bound(got, ref, bound, what="", slack=1.0):
    """Every element of |got - ref| within ``slack`` times an element-wise bound."""
    err = np.abs(np.asarray(got, np.float64) - ref)
    lim = slack * bound + 1e-6
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements outside the bound; "
                           f"worst excess {float((err - lim).max()):.3e}")


U_E4M3 = 2.0 ** -4
SUB_E4M3 = 2.0 ** -10
FP8_MFMA_ACC = 2.0 ** -11


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
    eta = 2.0 * FP8_MFMA_ACC * abs(scale) * (np.abs(q) @ np.abs(k).T).max(1)
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
