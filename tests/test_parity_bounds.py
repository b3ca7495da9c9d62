"""CPU checks of the element-wise bf16 rounding bound used by the backward
parity tests: a computation that performs exactly the roundings the bound
models stays inside it, and planted mistakes land far outside it."""

import numpy as np
import pytest
import torch

import oracle
from parity import bwd_error_bounds


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(torch.bfloat16).double().numpy()


def rounded_backward(q, k, v, do, scale, causal, mistake=None):
    """The backward with the bf16 roundings of the GPU arithmetic applied:
    O rounded before D, P rounded before dV, dS rounded before dK and dQ,
    outputs rounded once."""
    p, m, l = oracle.head_probabilities(q, k, scale, causal)
    o = bf(p @ v)
    dp = do @ v.T
    delta = (do * o).sum(1)
    ds = p * (dp - delta[:, None])
    dv = bf(bf(p).T @ do)
    dk = bf(scale * (bf(ds).T @ q))
    dq = bf(scale * (bf(ds) @ k))
    if mistake == "dk_no_transpose":
        dk = bf(scale * (bf(ds) @ q))
    if mistake == "dq_no_scale":
        dq = bf(bf(ds) @ k)
    if mistake == "dv_unrounded_delta_sign":
        dv = bf(bf(p).T @ -do)
    return dq, dk, dv


def args(n, d, seed, scale=None):
    g = np.random.default_rng(seed)
    arr = [bf(g.standard_normal((n, d))) for _ in range(4)]
    return (*arr, d ** -0.5 if scale is None else scale)


@pytest.mark.parametrize("n,d,causal,scale", [(2, 64, True, None), (64, 128, True, None),
                                              (150, 64, False, -0.3), (300, 32, False, None),
                                              (97, 16, True, 0.0)])
def test_rounded_computation_is_inside_bound(n, d, causal, scale):
    a = args(n, d, n + d, scale)
    ref = oracle.head_backward(*a, causal)
    got = rounded_backward(*a, causal)
    for g, r, b in zip(got, ref, bwd_error_bounds(*a, causal)):
        assert np.all(np.abs(g - r) <= b + 1e-6)


@pytest.mark.parametrize("mistake", ["dk_no_transpose", "dq_no_scale", "dv_unrounded_delta_sign"])
def test_planted_mistakes_break_bound(mistake):
    a = args(200, 64, 5)
    ref = oracle.head_backward(*a, False)
    got = rounded_backward(*a, False, mistake=mistake)
    worst = max(float((np.abs(g - r) / (b + 1e-6)).max())
                for g, r, b in zip(got, ref, bwd_error_bounds(*a, False)))
    assert worst > 10
