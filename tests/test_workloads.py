"""Host-side helpers: the memory arithmetic the explainer page prints, the
flop/byte counting, and the seeded input recipe."""

import json
import os

import numpy as np
import torch

from exact_io_aware_55_amd import inputs, workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_explainer_memory_arithmetic():
    with open(os.path.join(GOLDEN, "explainer_memory_arithmetic.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        if c["what"] == "score entries":
            got = workloads.score_entries(c["n"])
        elif c["what"].startswith("score bytes"):
            got = workloads.score_bytes(c["n"], c["elem_bytes"], c["heads"])
        elif c["what"] == "blocks along the sequence":
            got = c["n"] // c["block"]
        else:
            got = workloads.tile_bytes(c["rows"], c["cols"], c["elem_bytes"])
        assert got == c["exact"], c
    # "ueber 16 Millionen", "etwa 67 Millionen", "rund 128 MB", "ueber 4 GB", "512 MB"
    assert workloads.score_entries(4096) > 16e6
    assert abs(workloads.score_entries(8192) - 67e6) < 0.2e6
    assert workloads.score_bytes(8192, 2, 32) > 4 * 2 ** 30 - 1


def test_flop_counting():
    w = workloads.MHA_N4096_D128
    assert workloads.fwd_flops(w.B, w.H, w.N, w.d, False) == 4 * 4096 ** 2 * 128 * 128
    assert workloads.fwd_flops(w.B, w.H, w.N, w.d, True) == 2 * 4096 ** 2 * 128 * 128
    assert workloads.bwd_flops(4, 16, 4096, 64, True) == 2.5 * 2 * 4096 ** 2 * 64 * 64
    # sweep: fixed 16384 tokens, fwd = 1,048,576 N d
    for s in workloads.sweep(128):
        assert s.B * s.N == 16384
        assert workloads.fwd_flops(s.B, s.H, s.N, s.d, False) == 1048576 * s.N * s.d


def test_input_recipe_is_seeded_and_cast():
    a = inputs.make_qkv(1, 5, 2, 8, torch.bfloat16, seed=3, with_do=True)
    b = inputs.make_qkv(1, 5, 2, 8, torch.bfloat16, seed=3, with_do=True)
    for n in ("q", "k", "v", "do"):
        assert torch.equal(a[n], b[n]) and a[n].dtype == torch.bfloat16
    g = torch.Generator().manual_seed(3)
    q32 = torch.randn((1, 5, 2, 8), generator=g)
    assert torch.equal(a["q"], q32.to(torch.bfloat16))
    assert np.array_equal(inputs.to_f64(a["q"]), q32.to(torch.bfloat16).double().numpy())
    picks = inputs.pick_rows(2, 3, 50, 10)
    assert (0, 0, 0) in picks and (1, 2, 49) in picks and len(picks) >= 10
