"""CPU checks of the bf16 parity rule used by every GPU test (tests/parity.py).

The rule: every element within max(2e-2, min(W, 6 sigma)) and every tensor's
L2 error within max(5e-3 ||X*||, 1.5 sqrt(sum sigma^2)), where W and sigma
are the worst case and the standard deviation of the bf16 roundings the
kernels perform (P before P V and dV, dS before dK and dQ, the forward's O
before D, each output once).  These checks pin the rule to things other than
itself:

* a CPU computation with exactly those roundings (and fp64 elsewhere) passes
  at every shape the GPU tests use, and its errors never exceed the hard
  worst case W;
* the variance model is calibrated: the observed RMS error of that
  computation is a large fraction of sigma (not orders of magnitude below);
* at the benchmark shape the rule is the contract's fixed lines, unloosened;
* plausible kernel mistakes (untransposed dS, missing scale, sign flip, a
  skipped key block, a causal mask off by one, dropped row-statistic term)
  fail it."""

import numpy as np
import pytest
import torch

import oracle
import parity
from exact_io_aware_55_amd import inputs


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(torch.bfloat16).double().numpy()


def rounded(q, k, v, do, scale, causal, window=None, mistake=None):
    """Forward and backward with the bf16 roundings of the kernels applied:
    P rounded before P V and before dV, the forward's O rounded before
    D = rowsum(dO * O), dS rounded before dK and dQ, outputs rounded once."""
    p, _, _ = oracle.head_probabilities(q, k, scale, causal, window=window)
    if mistake == "skip_block":
        p = p.copy()
        p[:, 64:128] = 0.0
        p /= np.where(p.sum(1, keepdims=True) > 0, p.sum(1, keepdims=True), 1.0)
    if mistake == "causal_off_by_one":
        p, _, _ = oracle.head_probabilities(q, k, scale, False)
        vis = np.arange(q.shape[0])[None, :] <= np.arange(q.shape[0])[:, None] + 1
        p = np.where(vis, p, 0.0)
        p /= p.sum(1, keepdims=True)
    o = bf(bf(p) @ v)
    dp = do @ v.T
    delta = (do * o).sum(1)
    if mistake == "no_delta":
        delta = 0.0 * delta
    ds = p * (dp - delta[:, None])
    dv = bf(bf(p).T @ do)
    dk = bf(scale * (bf(ds).T @ q))
    dq = bf(scale * (bf(ds) @ k))
    if mistake == "dk_no_transpose":
        dk = bf(scale * (bf(ds) @ q))
    if mistake == "dq_no_scale":
        dq = bf(bf(ds) @ k)
    if mistake == "dv_sign":
        dv = -dv
    return {"O": o, "dQ": dq, "dK": dk, "dV": dv}


def head(n, d, seed, scale=None, h=0):
    x = inputs.make_qkv(1, n, h + 1, d, torch.bfloat16, seed=seed, with_do=True)
    q, k, v, do = (inputs.to_f64(x[name])[0, :, h] for name in ("q", "k", "v", "do"))
    return q, k, v, do, d ** -0.5 if scale is None else scale


SMALL = [(n, d, c) for d in (64, 128) for c in (False, True)
         for n in (1, 2, 7, 31, 64, 65, 127, 128, 129, 200, 513)]


@pytest.mark.parametrize("n,d,causal", SMALL, ids=[f"N{n}_d{d}_{'c' if c else 'nc'}" for n, d, c in SMALL])
def test_correct_rounding_passes_and_stays_inside_worst_case(n, d, causal):
    q, k, v, do, sc = head(n, d, seed=300 + n)
    terms, _ = parity.head_rounding_terms(q, k, v, sc, causal, do=do)
    got = rounded(q, k, v, do, sc, causal)
    for name, t in terms.items():
        parity.check_bf16(got[name], t, f"N{n} d{d} causal={causal} {name}")
        hard = parity.SECOND_ORDER * t.worst + parity.U_BF16 * np.abs(t.exact) + 1e-7
        assert np.all(np.abs(got[name] - t.exact) <= hard), name


@pytest.mark.parametrize("sc,causal,window", [(0.0, False, None), (-0.3, True, None), (0.7, True, None),
                                              (None, True, 1), (None, True, 100), (None, True, 129)])
def test_correct_rounding_passes_scales_and_windows(sc, causal, window):
    q, k, v, do, scale = head(300, 64, seed=17, scale=sc)
    terms, _ = parity.head_rounding_terms(q, k, v, scale, causal, window, do)
    got = rounded(q, k, v, do, scale, causal, window)
    for name, t in terms.items():
        parity.check_bf16(got[name], t, f"scale={scale} window={window} {name}")


def test_group_sums_pass_without_a_group_factor():
    """Grouped K/V heads: dK and dV of a K/V head sum the per-head
    gradients in fp32 and round once; the rule takes the sum of the heads'
    propagated terms and one output rounding (no factor of the group size)."""
    G, n, d, sc = 8, 256, 128, 128 ** -0.5
    x = inputs.make_qkv(1, n, G, d, torch.bfloat16, seed=41, with_do=True, H_kv=1)
    qn, kn, vn, dn = (inputs.to_f64(x[name]) for name in ("q", "k", "v", "do"))
    k, v = kn[0, :, 0], vn[0, :, 0]
    tk = tv = None
    dk_sum = dv_sum = 0.0
    for h in range(G):
        q, do = qn[0, :, h], dn[0, :, h]
        t, _ = parity.head_rounding_terms(q, k, v, sc, True, do=do)
        tk = t["dK"] if tk is None else tk + t["dK"]
        tv = t["dV"] if tv is None else tv + t["dV"]
        p, _, _ = oracle.head_probabilities(q, k, sc, True)
        o = bf(bf(p) @ v)
        ds = p * (do @ v.T - (do * o).sum(1)[:, None])
        dk_sum = dk_sum + sc * (bf(ds).T @ q)
        dv_sum = dv_sum + bf(p).T @ do
    parity.check_bf16(bf(dk_sum), tk, "group dK")
    parity.check_bf16(bf(dv_sum), tv, "group dV")


def test_variance_model_is_calibrated():
    """The observed L2 error of the correct rounding computation is between
    a quarter and all of the model's sqrt(sum sigma^2): the model is an upper
    bound (u^2/3 per rounding; round to nearest averages less) but not a
    vacuous one."""
    q, k, v, do, sc = head(1024, 128, seed=5)
    for causal in (False, True):
        terms, _ = parity.head_rounding_terms(q, k, v, sc, causal, do=do)
        got = rounded(q, k, v, do, sc, causal)
        for name, t in terms.items():
            sigma = np.sqrt((t.var + parity.VAR_U * t.exact ** 2).sum())
            ratio = np.linalg.norm(got[name] - t.exact) / sigma
            assert 0.25 < ratio < 1.0, (name, causal, ratio)


def test_rule_is_the_contract_at_the_benchmark_shape():
    """N = 4096, d = 128, non-causal (one head of the benchmark workload): no
    element gets a limit above 2e-2 and the L2 limit is 5e-3 ||X*||."""
    q, k, v, do, sc = head(4096, 128, seed=2)
    for name, t in parity.head_rounding_terms(q, k, v, sc, False, do=do)[0].items():
        elem, l2 = parity.rule_limits(t)
        assert np.all(elem == parity.TAU), name
        assert l2 == parity.RHO * np.linalg.norm(t.exact), name


@pytest.mark.parametrize("mistake,causal", [("dk_no_transpose", False), ("dq_no_scale", False),
                                            ("dv_sign", False), ("skip_block", False),
                                            ("causal_off_by_one", True), ("no_delta", False)])
def test_planted_mistakes_fail(mistake, causal):
    q, k, v, do, sc = head(200, 64, seed=5)
    terms, _ = parity.head_rounding_terms(q, k, v, sc, causal, do=do)
    got = rounded(q, k, v, do, sc, causal, mistake=mistake)
    failed = []
    for name, t in terms.items():
        try:
            parity.check_bf16(got[name], t, name)
        except AssertionError:
            failed.append(name)
    assert failed, f"{mistake} passed the rule"


def test_pooled_check_covers_every_head_and_group():
    """check_parity (the per-head thread pool the GPU tests call) on outputs
    of the rounding computation for a grouped shape: it passes, and a
    mistake planted in one query head of one group is found."""
    B, N, H, Hkv, d, sc = 2, 150, 4, 2, 64, 64 ** -0.5
    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=12, with_do=True, H_kv=Hkv)
    qn, kn, vn, dn = (inputs.to_f64(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = np.zeros_like(qn), np.zeros((B, H, N))
    dq, dk, dv = np.zeros_like(qn), np.zeros_like(kn), np.zeros_like(vn)
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hkv)
            args = (qn[b, :, h], kn[b, :, hk], vn[b, :, hk], dn[b, :, h], sc, True)
            r = rounded(*args)
            o[b, :, h], dq[b, :, h] = r["O"], r["dQ"]
            dk[b, :, hk] += r["dK"]
            dv[b, :, hk] += r["dV"]
            lse[b, h] = oracle.head_forward(*args[:3], sc, True)[1]
    summary = parity.check_parity(x, sc, True, o=o, lse=lse, grads=(dq, bf(dk), bf(dv)))
    assert {n: v["tensors"] for n, v in summary.items()} == {"O": 8, "dQ": 8, "dK": 4, "dV": 4}
    bad = dk.copy()
    bad[1, :, 1] += 0.05 * np.abs(bad[1, :, 1]).max()
    with pytest.raises(AssertionError, match=r"K/V head \(1, 1\) dK"):
        parity.check_parity(x, sc, True, grads=(dq, bf(bad), bf(dv)))
    lse_bad = lse.copy()
    lse_bad[0, 3, 7] += 2e-3
    with pytest.raises(AssertionError):
        parity.check_parity(x, sc, True, o=o, lse=lse_bad)


def test_sampled_rows_check():
    """check_rows_forward on sampled rows of the rounding computation passes,
    and a row taken from the wrong head fails."""
    B, N, H, d, sc = 1, 700, 2, 128, 128 ** -0.5
    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=13)
    qn, kn, vn = (inputs.to_f64(x[n]) for n in ("q", "k", "v"))
    picks = [(0, h, i) for h in range(H) for i in (0, 5, 129, 640, 699)]
    rows, lses = [], []
    for b, h, i in picks:
        p, m, l = oracle.head_probabilities(qn[b, :, h], kn[b, :, h], sc, True, rows=[i])
        rows.append(bf(bf(p) @ vn[b, :, h])[0])
        lses.append(m[0] + np.log(l[0]))
    parity.check_rows_forward(np.array(rows), np.array(lses), x, sc, True, picks)
    swapped = np.array(rows)
    swapped[[0, 5]] = swapped[[5, 0]]
    with pytest.raises(AssertionError):
        parity.check_rows_forward(swapped, np.array(lses), x, sc, True, picks)
