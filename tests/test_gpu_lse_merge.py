"""The (O, LSE) pair the forward writes is enough to combine attention over
separate key ranges, which is what spreading one long sequence over several
devices needs (the glossary page "Flash Attention", section "Flash Attention
и смежные понятия", ring attention: each device attends over its own block
of keys and values while the blocks travel around a ring).

On one GPU: the causal output for the queries in the second half of the
sequence is built from two independent forward calls over the two halves of
the keys, the first half unmasked (every one of those keys precedes those
queries) and the second half causal, and merged with
    LSE = log(exp(LSE_a) + exp(LSE_b)),
    O   = exp(LSE_a - LSE) O_a + exp(LSE_b - LSE) O_b.
The merged rows, and the first half's rows from a third call, are compared
with the oracle's full causal attention: every head within the fixed bf16
lines (max-abs 2e-2, relative L2 5e-3) and LSE within 1e-3.

The backward splits the same way: with the full sequence's O and LSE (what
the merge above yields), the backward of each (query half, key half) pair
that can see anything gives that pair's share of the gradients (P = exp(S -
LSE) and D = rowsum(dO * O) are row-global), and dQ of a query half is the
sum over its key halves, dK and dV of a key half the sum over its query
halves."""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_55_amd import inputs
from parity import LSE_MAX_ABS, max_abs, rel_l2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1024, 2000])
def test_causal_rows_from_two_key_halves(gpu_lib, N, d):
    B, H = 2, 4
    half = N // 2
    print(f"\n[lse merge] B{B} H{H} N{N} d{d}", flush=True)
    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=N + d)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    part = lambda t, lo, hi: t[:, lo:hi].contiguous()
    # queries [0, half) see only keys [0, half): one causal call
    o_1, l_1 = gpu_lib.forward(part(q, 0, half), part(k, 0, half), part(v, 0, half), causal=True)
    # queries [half, N): all keys [0, half) (unmasked) and keys [half, N) (causal)
    o_a, l_a = gpu_lib.forward(part(q, half, N), part(k, 0, half), part(v, 0, half), causal=False)
    o_b, l_b = gpu_lib.forward(part(q, half, N), part(k, half, N), part(v, half, N), causal=True)
    torch.cuda.synchronize()

    f64 = inputs.to_f64
    la, lb = f64(l_a), f64(l_b)                                 # [B, H, N - half]
    lse = np.logaddexp(la, lb)
    wa = np.exp(la - lse).transpose(0, 2, 1)[..., None]         # [B, N - half, H, 1]
    wb = np.exp(lb - lse).transpose(0, 2, 1)[..., None]
    o_2 = wa * f64(o_a) + wb * f64(o_b)
    o_all = np.concatenate([f64(o_1), o_2], axis=1)             # [B, N, H, d]
    l_all = np.concatenate([f64(l_1), lse], axis=2)             # [B, H, N]

    qn, kn, vn = (inputs.to_f64(x[n]) for n in ("q", "k", "v"))
    for b in range(B):
        for h in range(H):
            ro, rl = oracle.head_forward(qn[b, :, h], kn[b, :, h], vn[b, :, h], d ** -0.5, True)
            tag = f"N{N} d{d} head {(b, h)}"
            assert max_abs(o_all[b, :, h], ro) <= 2e-2, tag
            assert rel_l2(o_all[b, :, h], ro) <= 5e-3, tag
            assert max_abs(l_all[b, h], rl) <= LSE_MAX_ABS, tag


def half_spacing(x):
    """Half the bf16 spacing at each element of x (0 where x = 0): the most
    one rounding of a partial gradient to bf16 can move it."""
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1024, 2000])
def test_causal_gradients_from_query_and_key_halves(gpu_lib, N, d):
    """Three backward calls over the visible (query half, key half) pairs:
    (1, 1) causal, (2, 1) unmasked, (2, 2) causal.  The assembled dQ, dK, dV
    are held to the oracle's full causal backward within the fixed lines plus
    half a bf16 spacing of every partial that was rounded before the sum."""
    B, H = 2, 4
    half = N // 2
    print(f"\n[lse merge bwd] B{B} H{H} N{N} d{d}", flush=True)
    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=N + d + 7, with_do=True)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.forward(q, k, v, causal=True)
    rows = lambda t, lo, hi: t[:, lo:hi].contiguous()
    lrows = lambda lo, hi: lse[:, :, lo:hi].contiguous()
    h1, h2 = (0, half), (half, N)
    pair = lambda qh, kh, causal: gpu_lib.backward(rows(q, *qh), rows(k, *kh), rows(v, *kh), rows(o, *qh),
                                                   rows(do, *qh), lrows(*qh), causal=causal)
    dq11, dk11, dv11 = pair(h1, h1, True)
    dq21, dk21, dv21 = pair(h2, h1, False)
    dq22, dk22, dv22 = pair(h2, h2, True)
    torch.cuda.synchronize()

    f64 = inputs.to_f64
    parts = {
        "dq": ([f64(dq11)], [f64(dq21), f64(dq22)]),
        "dk": ([f64(dk11), f64(dk21)], [f64(dk22)]),
        "dv": ([f64(dv11), f64(dv21)], [f64(dv22)]),
    }
    got, slack = {}, {}
    for name, (first, second) in parts.items():
        got[name] = np.concatenate([sum(first), sum(second)], axis=1)          # [B, N, H, d]
        sl = lambda ps: sum(half_spacing(p) for p in ps) if len(ps) > 1 else np.zeros_like(ps[0])
        slack[name] = np.concatenate([sl(first), sl(second)], axis=1)
    qn, kn, vn, dn = (inputs.to_f64(x[n]) for n in ("q", "k", "v", "do"))
    for b in range(B):
        for h in range(H):
            ref = dict(zip(("dq", "dk", "dv"),
                           oracle.head_backward(qn[b, :, h], kn[b, :, h], vn[b, :, h], dn[b, :, h], d ** -0.5, True)))
            for name in ("dq", "dk", "dv"):
                g, r, sl = got[name][b, :, h], ref[name], slack[name][b, :, h]
                tag = f"N{N} d{d} head {(b, h)} {name}"
                assert np.all(np.abs(g - r) <= 2e-2 + sl), f"{tag}: max excess {np.max(np.abs(g - r) - sl):.3e}"
                assert np.linalg.norm(g - r) <= 5e-3 * np.linalg.norm(r) + np.linalg.norm(sl), tag


# ---------------------------------------------------------------------------
# fa_merge: the same merge on the GPU
# ---------------------------------------------------------------------------

def merge_inputs(B, N, H, d, seed):
    """Random O halves (bf16) and LSEs spread over +-30 with special rows:
    one range empty (LSE -inf, its O filled with NaN, which must not leak),
    both empty, a NaN LSE, and equal LSEs."""
    g = torch.Generator().manual_seed(seed)
    oa = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16)
    ob = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16)
    la = (torch.rand(B, H, N, generator=g) * 60 - 30).float()
    lb = (torch.rand(B, H, N, generator=g) * 60 - 30).float()
    la[0, 0, 1] = -float("inf")
    oa[0, 1, 0] = float("nan")
    lb[0, 0, 2] = -float("inf")
    ob[0, 2, 0] = float("nan")
    la[0, 0, 3] = lb[0, 0, 3] = -float("inf")
    la[0, 0, 4] = float("nan")
    lb[0, 0, 5] = la[0, 0, 5]
    return oa, la, ob, lb


def check_against_oracle_merge(got_o, got_l, oa, la, ob, lb):
    ro, rl = oracle.merge(inputs.to_f64(oa), inputs.to_f64(la), inputs.to_f64(ob), inputs.to_f64(lb))
    go, gl = inputs.to_f64(got_o), inputs.to_f64(got_l)
    # special rows: the same non-finite pattern as the oracle
    assert np.array_equal(np.isnan(gl), np.isnan(rl)) and np.array_equal(np.isinf(gl), np.isinf(rl))
    assert np.array_equal(np.isnan(go), np.isnan(ro))
    fin = np.isfinite(rl)
    assert np.all(np.abs(gl[fin] - rl[fin]) <= 1e-5 * np.maximum(1.0, np.abs(rl[fin])))
    ok = ~np.isnan(ro)
    # one bf16 rounding of an fp32 combination: half a spacing of the result,
    # plus fp32 slack relative to the two weighted terms (which can cancel):
    # w_a |O_a| + w_b |O_b| is the merge of the absolute values
    mag, _ = oracle.merge(np.abs(inputs.to_f64(oa)), inputs.to_f64(la), np.abs(inputs.to_f64(ob)),
                          inputs.to_f64(lb))
    assert np.all(np.abs(go[ok] - ro[ok]) <= half_spacing(ro[ok]) + 1e-6 * mag[ok] + 1e-30)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [6, 77, 1000])
def test_merge_kernel_matches_the_oracle_merge(gpu_lib, N, d):
    print(f"\n[fa_merge] B2 H3 N{N} d{d}", flush=True)
    oa, la, ob, lb = merge_inputs(2, N, 3, d, seed=N + d)
    dev = [t.to(DEV) for t in (oa, la, ob, lb)]
    o, lse = gpu_lib.merge(*dev)
    torch.cuda.synchronize()
    check_against_oracle_merge(o, lse, oa, la, ob, lb)
    # empty range: the other result exactly; both empty: zeros and -inf
    assert torch.equal(o[0, 1, 0].cpu(), ob[0, 1, 0]) and torch.equal(o[0, 2, 0].cpu(), oa[0, 2, 0])
    assert torch.all(o[0, 3, 0] == 0) and lse[0, 0, 3].item() == -float("inf")


def test_merge_in_place_is_the_same_merge(gpu_lib):
    """out = o_a and lse_out = lse_a (accumulation in place) give the same
    bits as a separate output."""
    print("\n[fa_merge] in place B2 H4 N513 d128", flush=True)
    oa, la, ob, lb = (t.to(DEV) for t in merge_inputs(2, 513, 4, 128, seed=9))
    o, lse = gpu_lib.merge(oa, la, ob, lb)
    oa2, la2 = oa.clone(), la.clone()
    o2, lse2 = gpu_lib.merge(oa2, la2, ob, lb, out=oa2, lse_out=la2)
    torch.cuda.synchronize()
    assert o2.data_ptr() == oa2.data_ptr() and lse2.data_ptr() == la2.data_ptr()
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16))
    assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32))


@pytest.mark.parametrize("d", [64, 128])
def test_merged_key_halves_on_the_gpu_are_causal_attention(gpu_lib, d):
    """The merge of the two forward calls of the test above, done by fa_merge
    in place, gives the oracle's full causal attention on every head."""
    B, H, N = 2, 4, 2000
    half = N // 2
    print(f"\n[fa_merge] causal halves B{B} H{H} N{N} d{d}", flush=True)
    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=31 + d)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    part = lambda t, lo, hi: t[:, lo:hi].contiguous()
    o_1, l_1 = gpu_lib.forward(part(q, 0, half), part(k, 0, half), part(v, 0, half), causal=True)
    o_a, l_a = gpu_lib.forward(part(q, half, N), part(k, 0, half), part(v, 0, half), causal=False)
    o_b, l_b = gpu_lib.forward(part(q, half, N), part(k, half, N), part(v, half, N), causal=True)
    gpu_lib.merge(o_a, l_a, o_b, l_b, out=o_a, lse_out=l_a)
    torch.cuda.synchronize()
    o_all = np.concatenate([inputs.to_f64(o_1), inputs.to_f64(o_a)], axis=1)
    l_all = np.concatenate([inputs.to_f64(l_1), inputs.to_f64(l_a)], axis=2)
    qn, kn, vn = (inputs.to_f64(x[n]) for n in ("q", "k", "v"))
    for b in range(B):
        for h in range(H):
            ro, rl = oracle.head_forward(qn[b, :, h], kn[b, :, h], vn[b, :, h], d ** -0.5, True)
            tag = f"d{d} head {(b, h)}"
            assert max_abs(o_all[b, :, h], ro) <= 2e-2, tag
            assert rel_l2(o_all[b, :, h], ro) <= 5e-3, tag
            assert max_abs(l_all[b, h], rl) <= LSE_MAX_ABS, tag


def test_shard_by_shard_accumulation_from_nothing(gpu_lib):
    """Four key quarters merged one by one into an accumulator that starts
    with LSE = -inf and uninitialised O (a range of weight 0 contributes
    nothing, whatever its O holds): non-causal attention over all keys."""
    B, H, N, d = 1, 4, 1024, 128
    print(f"\n[fa_merge] accumulate quarters B{B} H{H} N{N} d{d}", flush=True)
    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=41)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    acc_o = torch.full((B, N, H, d), float("nan"), device=DEV, dtype=torch.bfloat16)
    acc_l = torch.full((B, H, N), -float("inf"), device=DEV)
    # the forward takes N queries and N keys: each quarter's keys are tiled
    # four times and the scores of each copy shifted by -ln 4, so that the
    # four copies weigh as one
    quarter = N // 4
    for i in range(4):
        kq = k[:, i * quarter:(i + 1) * quarter].repeat(1, 4, 1, 1).contiguous()
        vq = v[:, i * quarter:(i + 1) * quarter].repeat(1, 4, 1, 1).contiguous()
        o_i, l_i = gpu_lib.forward(q, kq, vq, causal=False)
        l_i -= float(np.log(4.0))
        gpu_lib.merge(acc_o, acc_l, o_i, l_i, out=acc_o, lse_out=acc_l)
    torch.cuda.synchronize()
    qn, kn, vn = (inputs.to_f64(x[n]) for n in ("q", "k", "v"))
    go, gl = inputs.to_f64(acc_o), inputs.to_f64(acc_l)
    for h in range(H):
        ro, rl = oracle.head_forward(qn[0, :, h], kn[0, :, h], vn[0, :, h], d ** -0.5, False)
        assert max_abs(go[0, :, h], ro) <= 2e-2 and rel_l2(go[0, :, h], ro) <= 5e-3, h
        assert max_abs(gl[0, h], rl) <= LSE_MAX_ABS, h


def test_merge_full_size(gpu_lib):
    """B1 H32 N16384 d128 (the long causal workload's shape), every element
    against the oracle merge."""
    print("\n[fa_merge] B1 H32 N16384 d128", flush=True)
    oa, la, ob, lb = merge_inputs(1, 16384, 32, 128, seed=5)
    dev = [t.to(DEV) for t in (oa, la, ob, lb)]
    o, lse = gpu_lib.merge(*dev)
    torch.cuda.synchronize()
    check_against_oracle_merge(o, lse, oa, la, ob, lb)

