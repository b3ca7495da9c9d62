"""Workload catalogue and the work/traffic counting used by the bench.

Counting convention: the forward does 4*N*N*d flops per head (two N x N x d
products), the backward 2.5 times that (five such products, including the
recomputation of Q K^T that the pages note makes the total flop count slightly
higher; "Speicherbedarf und Laufzeitverhalten" on the explainer page), and a
causal mask halves both.

The bytes each kernel must move (the tensors that cross HBM at least once)
are counted per kernel in ``profiling.compulsory_bytes``.
"""

from __future__ import annotations

from dataclasses import dataclass, field


def score_entries(n: int) -> int:
    """Entries of one N x N score matrix (explainer page, introduction)."""
    return n * n


def score_bytes(n: int, elem_bytes: int = 2, heads: int = 1) -> int:
    """Bytes to materialise the N x N score matrix for ``heads`` heads."""
    return score_entries(n) * elem_bytes * heads


def tile_bytes(rows: int, cols: int, elem_bytes: int = 2) -> int:
    """Bytes of one rows x cols score tile (explainer page, "Tiling")."""
    return rows * cols * elem_bytes


def window_pairs(N: int, window: int) -> int:
    """Visible (query, key) pairs of one head under a causal sliding window:
    query i sees min(i + 1, window) keys."""
    w = min(window, N)
    return w * (w + 1) // 2 + (N - w) * w


def fwd_flops(B, H, N, d, causal, window=None):
    """Counted forward flops: 4 N^2 d per head, halved for causal (N^2 / 2
    pairs); with a sliding window, 4 d per visible pair."""
    f = 4.0 * N * N * d * B * H
    if window is not None:
        return 4.0 * d * window_pairs(N, window) * B * H
    return f / 2 if causal else f


def bwd_flops(B, H, N, d, causal, window=None):
    return 2.5 * fwd_flops(B, H, N, d, causal, window)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str            # "bf16" or "f32"
    seed: int
    backward: bool = False
    gain: float = 1.0
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)


# The five workloads of the method's evaluation (synthetic N(0,1) inputs).
SINGLE_HEAD_F32 = Workload("single_head_f32_n1024_d64", 1, 1, 1024, 64, False, "f32", 1,
                           note="fp32 path, K/V block 256")
MHA_N4096_D128 = Workload("mha_b4_h32_n4096_d128", 4, 32, 4096, 128, False, "bf16", 2)
MHA_N4096_D128_CAUSAL = Workload("mha_b4_h32_n4096_d128_causal", 4, 32, 4096, 128, True,
                                 "bf16", 2)
LONG_CAUSAL = Workload("long_b1_h32_n16384_d128_causal", 1, 32, 16384, 128, True, "bf16", 3)
BWD_CAUSAL_D64 = Workload("bwd_b4_h16_n4096_d64_causal", 4, 16, 4096, 64, True, "bf16", 4,
                          backward=True)


def sweep(d: int):
    """Fixed 16384 tokens per batch, H=16, non-causal, fwd+bwd."""
    out = []
    for n in (512, 1024, 2048, 4096, 8192, 16384):
        out.append(Workload(f"sweep_n{n}_d{d}", 16384 // n, 16, n, d, False, "bf16", 5,
                            backward=True))
    return out


ALL = [SINGLE_HEAD_F32, MHA_N4096_D128, MHA_N4096_D128_CAUSAL, LONG_CAUSAL, BWD_CAUSAL_D64]
