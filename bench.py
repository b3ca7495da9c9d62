"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch: the forward
(fa_fwd: tiled online softmax, writes O and LSE) followed by the backward by
recomputation as fa_bwd runs it (fa_bwd_dq_stats: dQ and the row statistics;
then fa_bwd_dkdv).
Default workload: B=4, H=32, N=4096, d=128, bf16, non-causal, scale 1/sqrt(d),
seeded N(0,1) inputs resident in HBM before timing starts.

Counted work: 4 N^2 d flops per head forward, 2.5x that backward, halved when
causal.  Peak: MI355X dense bf16 MFMA = 256 CU x 4096 flop/clk x 2.4 GHz =
2516.6 TFLOP/s.

Prints one JSON line (rank 0).  Beside the kernel it reports a naive
materialised-attention baseline on the same GPU (torch bf16 bmm + softmax,
scores and probabilities written to HBM, explicit backward) and the fp64 CPU
oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 5033.2     # dense fp8 MFMA: 256 CU x 8192 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--B", type=int, default=4)
    ap.add_argument("--H", type=int, default=32)
    ap.add_argument("--N", type=int, default=4096)
    ap.add_argument("--d", type=int, default=128)
    ap.add_argument("--causal", action="store_true")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--no-naive", action="store_true", help="skip the naive GPU baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (causal, long causal, d=64 causal)")
    ap.add_argument("--sweep", action="store_true",
                    help="run only the shape sweep at 16384 tokens (H=16, N 512..16384, d 64 and "
                         "128, non-causal, forward + backward) beside the naive GPU baseline")
    ap.add_argument("--mfma-calibration", action="store_true",
                    help="run only the matrix-core calibration kernel (pure bf16 MFMA, and with 2 or "
                         "4 vector instructions per MFMA) and print its sustained rates")
    ap.add_argument("--fp8-forward", action="store_true",
                    help="run only the FP8 forward workloads (E4M3; B4 H32 N4096 d128, and B1 H32 N16384 d128 causal) "
                         "and print their rates")
    ap.add_argument("--torch-sdpa-reference", action="store_true",
                    help="run only torch's scaled_dot_product_attention (flash and memory-efficient "
                         "backends) at --B/--H/--N/--d, both masks, as a reference beside the kernels")
    ap.add_argument("--mall-flush", action="store_true",
                    help="run only the cache-flush check: single fwd and fwd+bwd calls on "
                         "B4 H32 N4096 d128 and B1 H32 N16384 d128 causal, timed one by one, "
                         "with and without a 512 MiB overwrite between calls (outside the "
                         "timed region)")
    ap.add_argument("--lse-merge", action="store_true",
                    help="run only fa_merge (two attention results over disjoint key ranges "
                         "combined through their LSEs) at B1 H32 N16384 d128, apart and in place, "
                         "against the HBM bandwidth")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device-to-device copy of 1 GiB (3 times), the "
                         "reference for scaling HBM byte counters")
    return ap.parse_args()


def copy_calibration():
    """A plain 1 GiB device copy: reads 1 GiB and writes 1 GiB per launch."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 3}), flush=True)


# Matrix-core calibration: (label, workgroups of 4 waves, mode).  512
# workgroups is one full round at 2 waves per SIMD (as in the attention
# kernels); 256 is one wave per SIMD.  Modes: 0 constant operands, 1 random
# operands, 2 and 3 random plus 2 or 4 vector instructions per MFMA, 4 random
# with the A operand read from LDS.
MFMA_CALIBRATION = [("const_w2", 512, 0), ("random_w2", 512, 1), ("random_valu2_w2", 512, 2),
                    ("random_valu4_w2", 512, 3), ("random_lds_w2", 512, 4), ("random_w1", 256, 1),
                    ("const_w1", 256, 0), ("random_lds_valu4_w2", 512, 5), ("random_lds_valu4_w1", 256, 5),
                    ("random_lds_half_valu4_w2", 512, 6), ("random_lds_half_valu4_w1", 256, 6),
                    ("random_lds_valu2p5_w2", 512, 7), ("random_lds_valu2p5_w1", 256, 7)]


def torch_sdpa_reference(torch, B, H, N, d, seed):
    """torch's own scaled_dot_product_attention on the same shape, with each
    fused backend this build offers (flash, memory-efficient), forward alone
    and forward + backward, both masks: a reference from a production
    library on the same GPU, not part of the measured path."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    g = torch.Generator(device="cuda:0").manual_seed(seed)
    shape = (B, H, N, d)
    q, k, v, do = (torch.randn(shape, generator=g, device="cuda:0", dtype=torch.bfloat16) for _ in range(4))
    for t in (q, k, v):
        t.requires_grad_(True)
    out = {}
    for causal in (False, True):
        flops = 4.0 * N * N * d * B * H * (0.5 if causal else 1.0)
        for name, backend in (("flash", SDPBackend.FLASH_ATTENTION),
                              ("memory_efficient", SDPBackend.EFFICIENT_ATTENTION)):
            key = f"{name}_{'causal' if causal else 'noncausal'}"
            try:
                with sdpa_kernel(backend):
                    fwd = lambda: F.scaled_dot_product_attention(q, k, v, is_causal=causal)
                    step = lambda: fwd().backward(do)
                    fwd_ms, step_ms = median_ms(torch, fwd), median_ms(torch, step)
                out[key] = {"fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(flops / fwd_ms / 1e9, 1),
                            "fwd_bwd_ms": round(step_ms, 4),
                            "fwd_bwd_tflops": round(3.5 * flops / step_ms / 1e9, 1)}
            except Exception as exc:              # a backend this build lacks
                out[key] = {"error": str(exc)[:200]}
    return out


# Shapes for the cache-flush check: the headline shape and the long causal one.
FLUSH_WORKLOADS = [
    ("b4_h32_n4096_d128", 4, 32, 4096, 128, False),
    ("b1_h32_n16384_d128_causal", 1, 32, 16384, 128, True),
]
FLUSH_BYTES = 512 << 20          # twice the 256 MB Infinity Cache


def mall_flush(torch, binding, inputs, workloads, seed, reps=50, warmup=10):
    """Each call timed alone (events on the current stream around that call
    only), 50 reps after 10 warm-up calls, once back to back and once with a
    512 MiB buffer overwritten between calls so that neither L2 nor the
    Infinity Cache holds anything of the previous call.  The fill runs outside
    the events; a synchronisation after it keeps its tail out of the next
    call's time.  Reports medians and minima, and the median's change."""
    dev = torch.device("cuda:0")
    junk = torch.empty(FLUSH_BYTES // 4, device=dev, dtype=torch.float32)
    out = {}
    for name, B, H, N, d, causal in FLUSH_WORKLOADS:
        x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=seed, with_do=True)
        q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
        o, lse = binding.forward(q, k, v, causal=causal)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        ws = torch.empty(binding.bwd_workspace_size(B, H, N, d), device=dev, dtype=torch.uint8)
        _, calls = binding.backward_steps(q, k, v, o, do, lse, causal=causal, workspace=ws, out=grads)

        def fwd():
            binding.forward(q, k, v, causal=causal, out=o, lse=lse)

        def step():
            fwd()
            for c in calls:
                c()

        res = {}
        for tag, f, fl in (("fwd", fwd, workloads.fwd_flops(B, H, N, d, causal)),
                           ("fwd_bwd", step, workloads.fwd_flops(B, H, N, d, causal)
                            + workloads.bwd_flops(B, H, N, d, causal))):
            for flush in (False, True):
                for _ in range(warmup):
                    f()
                ms = []
                for r in range(reps):
                    if flush:
                        junk.fill_(float(r))
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    f()
                    e1.record()
                    torch.cuda.synchronize()
                    ms.append(e0.elapsed_time(e1))
                ms.sort()
                key = f"{tag}_{'flushed' if flush else 'warm'}"
                res[key] = {"median_ms": round(ms[reps // 2], 4), "min_ms": round(ms[0], 4),
                            "median_tflops": round(fl / (ms[reps // 2] * 1e-3) / 1e12, 1)}
            warm, cold = res[f"{tag}_warm"]["median_ms"], res[f"{tag}_flushed"]["median_ms"]
            res[f"{tag}_median_change"] = round(cold / warm - 1, 4)
        out[name] = res
        print(f"[mall flush] {name}: {json.dumps(res)}", file=sys.stderr, flush=True)
        del q, k, v, do, o, lse, grads, ws, calls
        torch.cuda.empty_cache()
    return out


# fa_merge: HBM-bound; its algorithmic bytes per launch read both O and both
# LSE arrays and write one of each.
MERGE_WORKLOAD = ("merge_b1_h32_n16384_d128", 1, 32, 16384, 128)


def lse_merge(torch, binding):
    """fa_merge at B1 H32 N16384 d128 (two 128 MiB bf16 O arrays and their
    LSEs), timed like the other workloads, apart and in place, against the
    HBM bandwidth (8 TB/s).  The counter-measured bytes per launch are
    reported when profiles/traffic.json holds them for these sources."""
    name, B, H, N, d = MERGE_WORKLOAD
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(3)
    oa, ob = (torch.randn(B, N, H, d, generator=g, device=dev).to(torch.bfloat16) for _ in range(2))
    la, lb = (torch.randn(B, H, N, generator=g, device=dev) * 4 for _ in range(2))
    o, lse = torch.empty_like(oa), torch.empty_like(la)
    algo = 3 * oa.numel() * 2 + 3 * la.numel() * 4
    out = {"workload": name, "algorithmic_bytes": algo}
    for tag, f in (("apart", lambda: binding.merge(oa, la, ob, lb, out=o, lse_out=lse)),
                   ("in_place", lambda: binding.merge(oa, la, ob, lb, out=oa, lse_out=la))):
        ms = median_ms(torch, f)
        gbps = algo / (ms * 1e-3) / 1e9
        out[tag] = {"ms": round(ms, 4), "gbps": round(gbps, 1), "frac_of_hbm": round(gbps / PEAK_HBM_GBS, 4)}
    out["traffic"] = measured_traffic("merge", name)
    # the practical HBM rate on the same GPU: torch's device copy of 256 MiB
    # (reads and writes 256 MiB each)
    src = torch.ones(1 << 28, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = median_ms(torch, lambda: dst.copy_(src))
    gbps = 2 * src.numel() / (ms * 1e-3) / 1e9
    out["copy_reference"] = {"ms": round(ms, 4), "gbps": round(gbps, 1), "frac_of_hbm": round(gbps / PEAK_HBM_GBS, 4)}
    return out


def mfma_calibration(torch, binding, iters=4000, launches=10):
    """Sustained rate of the calibration kernel (fa_calibrate_mfma): eight
    independent chains of 32x32x16 bf16 MFMAs per wave, back to back, against
    the nameplate dense bf16 peak.  A settling run first brings the clock to
    its sustained state."""
    o, _ = binding.calibrate_mfma(512, 4, iters, 1)
    for _ in range(20):
        binding.calibrate_mfma(512, 4, iters, 1, out=o)
    out = {}
    for label, n_wg, mode in MFMA_CALIBRATION:
        o, flops = binding.calibrate_mfma(n_wg, 4, iters, mode)
        for _ in range(2):
            binding.calibrate_mfma(n_wg, 4, iters, mode, out=o)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            binding.calibrate_mfma(n_wg, 4, iters, mode, out=o)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        tf = flops / (ms * 1e-3) / 1e12
        out[label] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    return out


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_io_aware_55_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# kernel name -> (sources that define it, how its algorithmic work is counted)
KERNELS = {
    "fwd": ("fa_fwd.hip", "fa_common.h", "fa_schedule.hip"),
    "bwd_dkdv": ("fa_bwd.hip", "fa_common.h", "fa_schedule.hip"),
    "bwd_dq": ("fa_bwd.hip", "fa_common.h", "fa_schedule.hip"),
    "merge": ("fa_merge.hip", "fa_common.h"),
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    absent or taken on a different version of the kernel's sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        table = json.load(fh)
    rec = table.get(f"{kernel}@{workload}")
    if not rec or rec.get("source_sha") != source_digest(*KERNELS[kernel]):
        return None
    return rec.get("bytes_per_launch")


def naive_step(torch, q, k, v, do, scale, causal):
    """Standard attention materialised in HBM (bf16), forward and backward."""
    B, N, H, d = q.shape
    bh = lambda t: t.permute(0, 2, 1, 3).reshape(B * H, N, d).contiguous()
    qh, kh, vh, doh = bh(q), bh(k), bh(v), bh(do)
    s = torch.bmm(qh, kh.transpose(1, 2).contiguous()) * scale
    if causal:
        s.masked_fill_(torch.ones(N, N, device=q.device, dtype=torch.bool).triu_(1), float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.bmm(p, vh)
    dv = torch.bmm(p.transpose(1, 2).contiguous(), doh)
    dp = torch.bmm(doh, vh.transpose(1, 2).contiguous())
    delta = (doh.float() * o.float()).sum(-1, keepdim=True)
    ds = (p.float() * (dp.float() - delta)).to(torch.bfloat16)
    dq = torch.bmm(ds, kh) * scale
    dk = torch.bmm(ds.transpose(1, 2).contiguous(), qh) * scale
    return o, dq, dk, dv


# Workloads reported beside the headline one (parity-test shapes of the
# same kernels): forward and backward timed separately, median of 5 samples
# of 10 back-to-back calls after 10 warm-up calls.
# (name, B, H, H_kv, N, d, causal, window): grouped-query attention with the
# pages' Llama 2 70B head counts (64 query heads over 8 K/V heads), and a
# causal sliding window of 4096 over 32768 tokens (the pages' Mistral 7B
# example; flops counted over the visible pairs only).
# b4_h16_n4096_d128 is the 16384-token sweep's N=4096, d=128 point, where the
# backward alone is held to 35% of the peak; b16_h16_n1024_d64 is a second
# sweep point.
EXTRA_WORKLOADS = [
    ("b4_h32_n4096_d128_causal", 4, 32, 32, 4096, 128, True, None),
    ("b4_h16_n4096_d128", 4, 16, 16, 4096, 128, False, None),
    ("b16_h16_n1024_d64", 16, 16, 16, 1024, 64, False, None),
    ("b1_h32_n16384_d128_causal", 1, 32, 32, 16384, 128, True, None),
    ("b4_h16_n4096_d64_causal", 4, 16, 16, 4096, 64, True, None),
    ("b2_h64_hkv8_n4096_d128_causal_gqa", 2, 64, 8, 4096, 128, True, None),
    ("b1_h32_n32768_d128_window4096", 1, 32, 32, 32768, 128, True, 4096),
]


def median_ms(torch, f, reps=10, samples=5, warmup=10):
    """Median over ``samples`` of the per-call time of ``reps`` back-to-back
    calls of f (events on the current stream), after ``warmup`` calls.  Two
    warm-up calls were too few: the first sample after them read up to 12%
    slow on a 0.55 ms kernel, later ones agreed within 1%."""
    for _ in range(warmup):
        f()
    ms = []
    for _ in range(samples):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / reps)
    return sorted(ms)[samples // 2]


def other_workloads(torch, binding, inputs, workloads, seed):
    out = {}
    dev = torch.device("cuda:0")
    for name, B, H, Hkv, N, d, causal, window in EXTRA_WORKLOADS:
        x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=seed, with_do=True, H_kv=Hkv)
        q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
        o, lse = binding.forward(q, k, v, causal=causal, window=window)
        if Hkv == H and window is None:
            _, calls = binding.backward_steps(q, k, v, o, do, lse, causal=causal)
        else:
            ws = torch.empty(binding.bwd_workspace_size(B, H, N, d), device=dev, dtype=torch.uint8)
            grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
            calls = [lambda: binding.backward(q, k, v, o, do, lse, causal=causal, workspace=ws,
                                              out=grads, window=window)]

        def fwd():
            binding.forward(q, k, v, causal=causal, out=o, lse=lse, window=window)

        def bwd():
            for c in calls:
                c()

        res = {}
        for tag, f, fl in (("fwd", fwd, workloads.fwd_flops(B, H, N, d, causal, window)),
                           ("bwd", bwd, workloads.bwd_flops(B, H, N, d, causal, window))):
            med = median_ms(torch, f)
            res[f"{tag}_ms"] = round(med, 4)
            res[f"{tag}_tflops"] = round(fl / (med * 1e-3) / 1e12, 1)
            res[f"{tag}_frac"] = round(fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if window is not None:
            res["pairs_skipped_frac"] = round(1 - workloads.window_pairs(N, window) / N ** 2, 4)
        out[name] = res
        del q, k, v, do, o, lse, calls
        torch.cuda.empty_cache()
    return out


# FP8 forward (fa_fwd_fp8, E4M3 inputs with per-head descales, bf16 O):
# forward only, timed like the other workloads, against the dense fp8 MFMA
# peak.
FP8_WORKLOADS = [
    ("b4_h32_n4096_d128_fp8", 4, 32, 32, 4096, 128, False, None),
    ("b1_h32_n16384_d128_causal_fp8", 1, 32, 32, 16384, 128, True, None),
]


def fp8_workloads(torch, binding, inputs, workloads, seed):
    out = {}
    dev = torch.device("cuda:0")
    for name, B, H, Hkv, N, d, causal, window in FP8_WORKLOADS:
        x = inputs.make_qkv_fp8(B, N, H, d, seed=seed, H_kv=Hkv)
        args = [x[n].to(dev) for n in ("q8", "k8", "v8", "q_descale", "k_descale", "v_descale")]
        o, lse = binding.forward_fp8(*args, causal=causal, window=window)
        med = median_ms(torch, lambda: binding.forward_fp8(*args, causal=causal, window=window,
                                                           out=o, lse=lse))
        tf = workloads.fwd_flops(B, H, N, d, causal, window) / (med * 1e-3) / 1e12
        out[name] = {"fwd_ms": round(med, 4), "fwd_tflops": round(tf, 1),
                     "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
        del args, o, lse
        torch.cuda.empty_cache()
    return out


# Shape sweep at a fixed 16384 tokens per batch: B = 16384 / N, H = 16,
# non-causal, forward + backward, each N beside the naive materialised
# attention on the same GPU.
SWEEP_N = (512, 1024, 2048, 4096, 8192, 16384)
SWEEP_D = (64, 128)


def shape_sweep(torch, binding, inputs, workloads, seed):
    rows = []
    dev = torch.device("cuda:0")
    for d in SWEEP_D:
        for N in SWEEP_N:
            B, H = 16384 // N, 16
            scale = d ** -0.5
            x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=seed, with_do=True)
            q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
            o, lse = binding.forward(q, k, v, causal=False)
            _, calls = binding.backward_steps(q, k, v, o, do, lse, causal=False)

            def fwd():
                binding.forward(q, k, v, causal=False, out=o, lse=lse)

            def step():
                fwd()
                for c in calls:
                    c()

            fwd_fl = workloads.fwd_flops(B, H, N, d, False)
            bwd_fl = workloads.bwd_flops(B, H, N, d, False)
            f_ms = median_ms(torch, fwd)
            s_ms = median_ms(torch, step)
            row = {"N": N, "B": B, "H": H, "d": d,
                   "fwd_ms": round(f_ms, 4), "fwd_tflops": round(fwd_fl / (f_ms * 1e-3) / 1e12, 1),
                   "fwd_bwd_ms": round(s_ms, 4),
                   "fwd_bwd_tflops": round((fwd_fl + bwd_fl) / (s_ms * 1e-3) / 1e12, 1)}
            try:
                n_ms = median_ms(torch, lambda: naive_step(torch, q, k, v, do, scale, False),
                                 reps=2, samples=3, warmup=2)
                row["naive_fwd_bwd_ms"] = round(n_ms, 3)
                row["naive_fwd_bwd_tflops"] = round((fwd_fl + bwd_fl) / (n_ms * 1e-3) / 1e12, 1)
                row["speedup_over_naive"] = round(n_ms / s_ms, 2)
            except RuntimeError as exc:   # out of memory for the materialised matrices
                row["naive_error"] = str(exc)[:120]
            print(json.dumps({"sweep_row": row}), file=sys.stderr, flush=True)
            rows.append(row)
            del x, q, k, v, do, o, lse, calls
            torch.cuda.empty_cache()
    return rows


def cpu_baseline(x, args, flops_per_head):
    """fp64 oracle (forward + backward per head) on a bounded sample of heads."""
    import numpy as np
    import threadpoolctl

    import oracle
    from exact_io_aware_55_amd import inputs

    qn, kn, vn, dn = (inputs.to_f64(x[n]) for n in ("q", "k", "v", "do"))
    scale = args.d ** -0.5
    heads = [(b, h) for b in range(args.B) for h in range(args.H)]
    done = 0
    t0 = time.perf_counter()
    for b, h in heads:
        a = (qn[b, :, h], kn[b, :, h], vn[b, :, h])
        oracle.head_forward(*a, scale, args.causal)
        oracle.head_backward(*a, dn[b, :, h], scale, args.causal)
        done += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    el = time.perf_counter() - t0
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    return {
        "value": flops_per_head * done / el / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} heads (fp64 forward + backward per head, N={args.N}, "
                  f"d={args.d}, causal={args.causal}) in {el:.1f} s; BLAS threads={threads}, "
                  f"host cpus={os.cpu_count()}",
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: every (batch, head) is independent and the library "
              "has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    sys.path.insert(0, ROOT)
    from exact_io_aware_55_amd import binding, inputs, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    if args.mfma_calibration:
        print(json.dumps({"mfma_calibration": mfma_calibration(torch, binding),
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}), flush=True)
        return
    if args.torch_sdpa_reference:
        print(json.dumps({"torch_sdpa_reference": torch_sdpa_reference(torch, args.B, args.H, args.N, args.d,
                                                                       args.seed),
                          "config": {"workload": f"b{args.B}_h{args.H}_n{args.N}_d{args.d}"},
                          "unit": "TFLOP/s", "dtype": "bf16"}), flush=True)
        return
    if args.mall_flush:
        print(json.dumps({"mall_flush": mall_flush(torch, binding, inputs, workloads, args.seed),
                          "flush_bytes": FLUSH_BYTES, "unit": "ms", "dtype": "bf16"}), flush=True)
        return
    if args.lse_merge:
        print(json.dumps({"lse_merge": lse_merge(torch, binding), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "dtype": "bf16"}), flush=True)
        return
    if args.fp8_forward:
        print(json.dumps({"fp8_forward": fp8_workloads(torch, binding, inputs, workloads, args.seed),
                          "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s"}), flush=True)
        return
    if args.sweep:
        rows = shape_sweep(torch, binding, inputs, workloads, args.seed)
        print(json.dumps({"metric": "attention TFLOP/s (fwd+bwd) bf16, shape sweep at 16384 tokens",
                          "unit": "TFLOP/s", "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": "sweep_16384_tokens_h16_noncausal"},
                          "sweep": rows}), flush=True)
        return
    dev = torch.device("cuda:0")
    B, H, N, d, causal = args.B, args.H, args.N, args.d, args.causal
    scale = d ** -0.5
    wl = f"b{B}_h{H}_n{N}_d{d}{'_causal' if causal else ''}_fwd_bwd"

    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=args.seed, with_do=True)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(binding.bwd_workspace_size(B, H, N, d), device=dev, dtype=torch.uint8)

    def fwd():
        binding.forward(q, k, v, causal=causal, scale=scale, out=o, lse=lse)

    fwd()
    _, bwd_calls = binding.backward_steps(q, k, v, o, do, lse, causal=causal, scale=scale,
                                          workspace=ws, out=(dq, dk, dv))
    stages = [("fwd", fwd)] + list(zip(("bwd_dq", "bwd_dkdv"), bwd_calls))
    for _ in range(args.warmup):
        for _, f in stages:
            f()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for j, (_, f) in enumerate(stages):
            f()
            ev[s][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {name: sum(ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(args.steps)) / args.steps
           for j, (name, _) in enumerate(stages)}
    fwd_fl = workloads.fwd_flops(B, H, N, d, causal)
    bwd_fl = workloads.bwd_flops(B, H, N, d, causal)
    step_fl = fwd_fl + bwd_fl
    ms_per_step = wall / args.steps * 1e3
    value = step_fl / (ms_per_step * 1e-3) / 1e12

    rows = B * H * N
    # Work each kernel must do in this design.  The backward splits into a
    # key-block kernel (S, dP, dV, dK: 8 N^2 d per head) and a query-block
    # kernel (S, dP, dQ: 6 N^2 d per head); the metric itself counts the
    # backward as 10 N^2 d per head (2.5x the forward), so the two kernels
    # execute 1.4x the counted backward work.
    half = 0.5 if causal else 1.0
    algo = {
        "fwd": ("mfma", fwd_fl),
        "bwd_dkdv": ("mfma", 8.0 * N * N * d * B * H * half),
        "bwd_dq": ("mfma", 6.0 * N * N * d * B * H * half),
    }
    kernels = {}
    for name, ms in per.items():
        bound, work = algo[name]
        if bound == "mfma":
            ach = work / (ms * 1e-3) / 1e12
            kernels[name] = {"ms": round(ms, 4), "tflops": round(ach, 1),
                             "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        else:
            ach = work / (ms * 1e-3) / 1e9
            kernels[name] = {"ms": round(ms, 4), "gbs": round(ach, 1),
                             "frac": round(ach / PEAK_HBM_GBS, 4)}
    dom = max(per, key=per.get)
    bound, work = algo[dom]
    if bound == "mfma":
        ach, peak, unit = work / (per[dom] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        ach, peak, unit = work / (per[dom] * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"bound": bound, "kernel": dom, "achieved": round(ach, 2), "peak": peak,
                "unit": unit, "frac": round(ach / peak, 4),
                "traffic": measured_traffic(dom, wl)}

    out = {
        "metric": "attention TFLOP/s (fwd+bwd) bf16 N=4096 d=128 on 1 GPU; % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                   "layout": "[B,N,H,d]", "scale": "1/sqrt(d)", "parallelism": "single GPU"},
        "fwd_tflops": round(fwd_fl / (per["fwd"] * 1e-3) / 1e12, 1),
        "bwd_tflops": round(bwd_fl / (sum(per[n] for n in per if n != "fwd") * 1e-3) / 1e12, 1),
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "kernels": kernels,
        "roofline": roofline,
    }

    if not args.no_extra:
        out["other_workloads"] = other_workloads(torch, binding, inputs, workloads, args.seed)
        out["fp8_forward"] = fp8_workloads(torch, binding, inputs, workloads, args.seed)
        out["lse_merge"] = lse_merge(torch, binding)
        torch.cuda.empty_cache()
        out["mfma_calibration"] = mfma_calibration(torch, binding, launches=4)

    if not args.no_naive:
        try:
            for _ in range(2):
                naive_step(torch, q, k, v, do, scale, causal)
            torch.cuda.synchronize()
            reps = max(3, min(10, args.steps))
            t1 = time.perf_counter()
            for _ in range(reps):
                naive_step(torch, q, k, v, do, scale, causal)
            torch.cuda.synchronize()
            nms = (time.perf_counter() - t1) / reps * 1e3
            out["naive_gpu_baseline"] = {
                "value": round(step_fl / (nms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "ms_per_step": round(nms, 3),
                "kind": "torch bf16 materialised scores + softmax + explicit backward",
                "speedup_of_kernel": round(nms / ms_per_step, 2)}
        except RuntimeError as exc:   # e.g. out of memory at very large shapes
            out["naive_gpu_baseline"] = {"error": str(exc)[:200]}
        torch.cuda.empty_cache()

    if not args.no_cpu:
        per_head = (fwd_fl + bwd_fl) / (B * H)
        out["cpu_baseline"] = cpu_baseline(x, args, per_head)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
