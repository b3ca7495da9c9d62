"""Plain fp64 CPU oracle for exact (FlashAttention) attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.
The product path (the HIP library and its Python binding) never touches it,
and this module imports nothing from that path: it takes numpy arrays and
returns numpy arrays.

What it computes is the *definition* of attention, not the tiled algorithm.
The pages state that the tiled method is exact up to floating-point rounding
("FlashAttention" explainer, sections "Speicherbedarf und Laufzeitverhalten"
and "Grenzen und Einschraenkungen"; glossary page, introduction), so the plain
definition is the right reference:

* scores  S = scale * Q K^T  (glossary page, "How it works", the standard
  attention line of its PyTorch sketch; the 1/sqrt(d) scale is the pages'
  choice and is an argument here),
* optional causal mask: query i sees key j only when j <= i (the pages name
  causal vs. bidirectional masks in the "Grenzen, Stolpersteine" section of the
  kernel-engineering page without defining it; lower-triangular is the
  reading taken),
* softmax over the whole row, done in two passes (row max, then exponentials
  and their sum), the numerically stable form the pages describe,
* O = P V, and the per-row statistics exported as one log-sum-exp
  LSE = m + ln(l) (the pages keep the row maximum and the row sum; LSE carries
  the same information, P = exp(S - LSE)).

The pages give no backward formula; they only say that the backward pass
recomputes the scores from Q and K rather than storing an N x N matrix
(explainer, "Recomputation beim Rueckwaertsdurchlauf"; glossary "How it
works").  The oracle uses the textbook
softmax Jacobian:

    dV = P^T dO,  dP = dO V^T,  Delta_i = sum_j P_ij dP_ij,
    dS = P * (dP - Delta),  dQ = scale * dS K,  dK = scale * dS^T Q.

Delta is taken in its definition form (a row sum over the N x N product); the
GPU path uses the equivalent row dot product of dO and O.

Tensors use the [B, N, H, d] layout; LSE uses [B, H, N].

Sliding-window attention (same page and section, subsection "Sliding Window
Attention": each position attends to a fixed neighbourhood).  The page gives
a window size of 4096 tokens for its causal language-model example without
saying whether the window counts the query itself; the reading taken is
causal with the window counting it: query i sees keys j with
i - window < j <= i.

Grouped-query attention (explainer page "Flash Attention", section "Varianten
und Erweiterungen", subsection "Grouped Query Attention": several query heads
share one K/V group): K and V may have H_kv heads with H a multiple of H_kv.
The page does not say which query heads form a group; the reading taken is
contiguous groups, query head h reading K/V head h // (H / H_kv).  Each query
head is then ordinary attention against its group's K and V, and the gradient
of a shared K/V head is the sum of its query heads' gradients (the chain rule
over a tensor used G times).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head",
    "head_forward",
    "head_backward",
    "head_forward_blockwise",
    "head_probabilities",
    "forward",
    "backward",
    "forward_rows",
]


def _f64(x):
    """Upcast any float array (fp32, bf16-as-fp32, fp64) to fp64 exactly."""
    return np.asarray(x, dtype=np.float64)


def _visible(nq: int, nk: int, causal: bool, rows=None, window=None):
    """Boolean mask [len(rows), nk]: True where query row i may see key j.

    Causal means key j is visible to query i when j <= i (square N x N case).
    A sliding window (causal only) further requires j > i - window: each
    query sees its own key and the window - 1 keys before it.
    """
    r = np.arange(nq) if rows is None else np.asarray(rows)
    if not causal:
        if window is not None:
            raise ValueError("a sliding window is defined for causal attention only")
        return np.ones((r.shape[0], nk), dtype=bool)
    j = np.arange(nk)[None, :]
    vis = j <= r[:, None]
    if window is not None:
        if window < 1:
            raise ValueError("window must be >= 1")
        vis &= j > r[:, None] - window
    return vis


def head_probabilities(q, k, scale, causal, rows=None, window=None):
    """Return (P, m, l) for one head by the two-pass softmax of the definition.

    q: [Nq, d], k: [Nk, d].  ``rows`` optionally selects query rows (absolute
    indices, used by the causal mask).  Masked scores are -inf, so their
    probability is exactly 0.
    """
    q = _f64(q)
    k = _f64(k)
    nq = q.shape[0]
    if rows is not None:
        q = q[np.asarray(rows)]
    s = scale * (q @ k.T)
    s = np.where(_visible(nq, k.shape[0], causal, rows, window), s, -np.inf)
    # pass 1: row maximum
    m = s.max(axis=1)
    # pass 2: exponentials relative to the maximum, and their sum
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def head_forward(q, k, v, scale, causal, rows=None, window=None):
    """One head: O = softmax(scale Q K^T [masked]) V and LSE = m + ln l.

    Returns (O [len(rows) or N, d], LSE [len(rows) or N]) in fp64.
    """
    p, m, l = head_probabilities(q, k, scale, causal, rows, window)
    o = p @ _f64(v)
    lse = m + np.log(l)
    return o, lse


def head_backward(q, k, v, do, scale, causal, window=None):
    """One head: (dQ, dK, dV) of L = sum(O * dO) by the softmax Jacobian.

    P is recomputed from the definition (no stored N x N from a forward).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    p, _, _ = head_probabilities(q, k, scale, causal, window=window)
    dv = p.T @ do
    dp = do @ v.T
    delta = (p * dp).sum(axis=1)          # definition form of Delta_i
    ds = p * (dp - delta[:, None])        # masked entries: p == 0 -> ds == 0
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def head_forward_blockwise(q, k, v, scale, causal, block, dtype=np.float64, window=None):
    """The tiled online-softmax forward over key/value blocks, for self-tests.

    This follows the streaming description on the glossary page ("How it
    works"): for each key/value block compute the scores, raise the running
    row maximum, rescale the running sum and the partial output by
    exp(old max - new max), add the block's exponentials and their product
    with V, and divide by the running sum once at the end.  ``dtype`` selects
    the arithmetic precision (fp64 by default, fp32 to reproduce the page's
    worked example).  It is never used to check the GPU; it pins the claim
    that the blockwise result equals the full softmax.  With a sliding
    ``window`` a block no row can see is skipped without being read, as the
    page describes ("Sliding Window Attention"); the number of skipped blocks
    is stored in the function attribute ``skipped``.
    """
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    n, d = q.shape
    nk = k.shape[0]
    sc = dtype(scale)
    vis_all = _visible(n, nk, causal, window=window)
    o = np.zeros((n, v.shape[1]), dtype=dtype)
    lse = np.zeros(n, dtype=dtype)
    largest_tile = (0, 0)
    skipped = 0
    # the page's sketch streams K/V blocks past all queries at once; with a
    # window the queries go in blocks of the same size too, so that whole
    # (query block, key block) tiles outside every window can be skipped
    qblock = block if window is not None else n
    for qs in range(0, n, qblock):
        qb = q[qs:qs + qblock]
        run_max = np.full((qb.shape[0], 1), -np.inf, dtype=dtype)
        run_sum = np.zeros((qb.shape[0], 1), dtype=dtype)
        acc = np.zeros((qb.shape[0], v.shape[1]), dtype=dtype)
        for start in range(0, nk, block):
            vis = vis_all[qs:qs + qblock, start:start + block]
            if window is not None and not vis.any():
                skipped += 1          # a block outside every row's window: never read
                continue
            kb = k[start:start + block]
            vb = v[start:start + block]
            s = (qb @ kb.T) * sc
            largest_tile = max(largest_tile, s.shape)
            if causal:
                s = np.where(vis, s, dtype(-np.inf))
            blk_max = s.max(axis=1, keepdims=True)
            new_max = np.maximum(run_max, blk_max)
            # a row that has seen no visible key yet keeps max -inf; subtract 0
            safe = np.where(np.isfinite(new_max), new_max, dtype(0))
            alpha = np.exp(run_max - safe)
            p = np.exp(s - safe)
            run_sum = run_sum * alpha + p.sum(axis=1, keepdims=True)
            acc = acc * alpha + p @ vb
            run_max = new_max
        o[qs:qs + qblock] = acc / run_sum
        lse[qs:qs + qblock] = (run_max + np.log(run_sum))[:, 0]
    head_forward_blockwise.skipped = skipped
    return o, lse, largest_tile


def kv_head(h, H, H_kv):
    """K/V head read by query head h (contiguous groups of H / H_kv)."""
    if H_kv < 1 or H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    return h // (H // H_kv)


def _heads_of(b, h, heads):
    if heads is None:
        return [(bi, hi) for bi in range(b) for hi in range(h)]
    return [tuple(x) for x in heads]


def forward(q, k, v, scale, causal, heads=None, window=None):
    """[B,N,H,d] forward.  Returns O [B,N,H,d] and LSE [B,H,N] in fp64.

    ``heads`` optionally restricts the work to a list of (b, h) pairs; the
    other entries of the outputs are NaN.
    """
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    o = np.full((B, N, H, v.shape[3]), np.nan)
    lse = np.full((B, H, N), np.nan)
    for b, h in _heads_of(B, H, heads):
        g = kv_head(h, H, Hkv)
        oh, lh = head_forward(q[b, :, h, :], k[b, :, g, :], v[b, :, g, :], scale, causal,
                              window=window)
        o[b, :, h, :] = oh
        lse[b, h, :] = lh
    return o, lse


def forward_rows(q, k, v, scale, causal, picks, window=None):
    """Forward for selected query rows only.

    ``picks`` is a list of (b, h, i).  Returns (O rows [len, d], LSE [len]).
    Each row depends only on its query and the visible keys of its head, so
    this is the definition evaluated row by row; used to sample outputs of
    workloads too large for a full fp64 N x N per head.
    """
    out_o = []
    out_l = []
    H, Hkv = q.shape[2], k.shape[2]
    for b, h, i in picks:
        g = kv_head(h, H, Hkv)
        oh, lh = head_forward(q[b, :, h, :], k[b, :, g, :], v[b, :, g, :], scale, causal,
                              rows=[i], window=window)
        out_o.append(oh[0])
        out_l.append(lh[0])
    return np.array(out_o), np.array(out_l)


def backward(q, k, v, do, scale, causal, heads=None, window=None):
    """Backward.  Returns dQ ([B,N,H,d]), dK and dV (shaped like k and v) in
    fp64.  With grouped K/V heads a K/V head's gradient sums over its query
    heads.

    ``heads`` optionally restricts the work to a list of (b, h) pairs; entries
    no listed head touches are NaN.
    """
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    for b, h in _heads_of(B, H, heads):
        g = kv_head(h, H, Hkv)
        a, bb, c = head_backward(q[b, :, h, :], k[b, :, g, :], v[b, :, g, :],
                                 do[b, :, h, :], scale, causal, window)
        dq[b, :, h, :] = a
        if np.isnan(dk[b, 0, g, 0]):
            dk[b, :, g, :] = 0.0
            dv[b, :, g, :] = 0.0
        dk[b, :, g, :] += bb
        dv[b, :, g, :] += c
    return dq, dk, dv


def merge(o_a, lse_a, o_b, lse_b):
    """Attention over the union of two disjoint key ranges, from the results
    over each range: the running-maximum rescaling of the explainer's
    "Tiling" section (and the glossary's online softmax) applied once to two
    finished blocks.  With L = log(exp(LSE_a) + exp(LSE_b)),

        O = exp(LSE_a - L) O_a + exp(LSE_b - L) O_b,   LSE = L.

    o_a, o_b: [B, N, H, d]; lse_a, lse_b: [B, H, N].  A range of weight 0
    (LSE -inf) contributes nothing, whatever its O holds; a row that sees no
    key in either range (both LSEs -inf) gets O = 0 and LSE = -inf; NaN in an
    LSE propagates to its row.  Returns fp64 (O, LSE)."""
    la, lb = _f64(lse_a), _f64(lse_b)
    m = np.maximum(la, lb)                    # NaN in either stays NaN
    empty = m == -np.inf
    ms = np.where(empty, 0.0, m)
    ea, eb = np.exp(la - ms), np.exp(lb - ms)
    tot = np.where(empty, 1.0, ea + eb)
    lse = np.where(empty, -np.inf, ms + np.log(tot))
    wa = np.where(empty, 0.0, ea / tot).transpose(0, 2, 1)[..., None]   # [B, N, H, 1]
    wb = np.where(empty, 0.0, eb / tot).transpose(0, 2, 1)[..., None]
    ta = np.where(wa == 0, 0.0, wa * _f64(o_a))
    tb = np.where(wb == 0, 0.0, wb * _f64(o_b))
    return ta + tb, lse

