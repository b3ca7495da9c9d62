"""Turns rocprofv3 output of ``bench.py`` runs into the text summaries kept
under ``profiles/`` (a kernel-trace table and an HBM-traffic table plus the
``traffic.json`` that ``bench.py`` reads for its roofline ``traffic`` field),
and the growth of those bytes with the sequence length (``scaling``).

Usage, from the repository root, after the rocprofv3 runs listed in each
summary::

    python -m exact_io_aware_55_amd.profiling trace DIR OUT.md TITLE COMMAND
    python -m exact_io_aware_55_amd.profiling traffic FETCH WRITE COPY_FETCH COPY_WRITE OUT.md WORKLOAD
    python -m exact_io_aware_55_amd.profiling counters MFMA_DIR LDS_DIR TRACE_DIR OUT.md WORKLOAD [BENCH_ARGS]
    python -m exact_io_aware_55_amd.profiling scaling COPY_FETCH COPY_WRITE OUT.md B H d N:FETCH:WRITE ...
    python -m exact_io_aware_55_amd.profiling valu VALU_DIR TRACE_DIR OUT.md WORKLOAD [BENCH_ARGS]
    python -m exact_io_aware_55_amd.profiling calibration RATES.json MFMA_DIR OUT.md

``DIR`` holds a ``--kernel-trace --stats`` run (``*_kernel_stats.csv``); the
traffic arguments are the output folders of four ``--pmc`` runs: FETCH_SIZE
and WRITE_SIZE of the bench workload, and the same two counters for the
``bench.py --copy-calibration`` device copy of 1 GiB, whose known byte count
scales the counters to bytes.  ``counters`` summarises two more ``--pmc``
runs: matrix-core busy cycles and bf16 MFMA operations, and LDS bank / address
conflicts and LDS activity.  ``valu`` summarises the vector-instruction group
(vector, transcendental, MFMA and LDS instructions, MFMA/vector co-execution
and wave waiting cycles) per kernel; ``calibration`` the matrix-core
calibration kernel's rates (the JSON line of ``bench.py --mfma-calibration``)
beside its clock and MFMA-busy counters.
"""
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# bench.py stage -> (kernel symbol prefix, sources that define it)
STAGES = {
    "fwd": ("fa::fwd_bf16_kernel", ("fa_fwd.hip", "fa_common.h", "fa_schedule.hip")),
    "bwd_preprocess": ("fa::bwd_pre_kernel", ("fa_bwd.hip", "fa_common.h")),
    "bwd_dkdv": ("fa::bwd_dkdv_kernel", ("fa_bwd.hip", "fa_common.h", "fa_schedule.hip")),
    "bwd_dq": ("fa::bwd_dq_kernel", ("fa_bwd.hip", "fa_common.h", "fa_schedule.hip")),
    "merge": ("fa::merge_kernel", ("fa_merge.hip", "fa_common.h")),
}


def source_digest(names):
    """Same digest as bench.py: sha256 of the kernel's sources, 16 hex digits."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_io_aware_55_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _one(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def _short(name):
    """Kernel name without its return type and parameter list.  A name the
    profiler left mangled (fa::<ident><integer or bool template arguments>)
    is read into the same form."""
    m = re.match(r"_ZN2fa(\d+)", name)
    if m:
        n = int(m.group(1))
        ident, rest = name[m.end():m.end() + n], name[m.end() + n:]
        t = re.match(r"I((?:L[ib]\d+E)+)E", rest)
        args = ""
        if t:
            vals = [("true" if v == "1" else "false") if k == "b" else v
                    for k, v in re.findall(r"L([ib])(\d+)E", t.group(1))]
            args = "<" + ", ".join(vals) + ">"
        return f"fa::{ident}{args}"
    return name.split("(")[0].replace("void ", "").strip()


def trace(folder, out, title, command):
    rows = list(csv.DictReader(open(_one(os.path.join(folder, "**", "*kernel_stats.csv")))))
    lines = [f"# {title}", "", "Command (from the repository root on one MI355X, after "
             "`cd /tmp && export TMPDIR=/tmp`; `$REPO` is the repository root, `$OUT` the folder "
             "that receives the profiler output):", "",
             "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _counter(folder):
    """kernel name -> mean counter value per dispatch (KiB)."""
    acc = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def traffic(fetch, write, copy_fetch, copy_write, out, workload, compulsory=None):
    f, w = _counter(fetch), _counter(write)
    cf, cw = _counter(copy_fetch), _counter(copy_write)
    copy = [k for k in cf if "copy" in k.lower()][0]
    gib_kib = (1 << 30) / 1024
    fs, ws = gib_kib / cf[copy], gib_kib / cw[copy]
    table_path = os.path.join(os.path.dirname(out), "traffic.json")
    table = json.load(open(table_path)) if os.path.exists(table_path) else {}
    lines = []
    for stage, (prefix, srcs) in STAGES.items():
        names = [k for k in f if k.startswith(prefix)]
        if not names:
            continue
        k = names[0]
        rd, wr = f[k] * fs * 1024, w.get(k, 0.0) * ws * 1024
        table[f"{stage}@{workload}"] = {
            "kernel": k, "bytes_per_launch": int(rd + wr), "read_bytes": int(rd),
            "written_bytes": int(wr), "fetch_kib": f[k], "write_kib": w.get(k, 0.0),
            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
            "source_sha": source_digest(srcs)}
        comp = (compulsory or {}).get(stage)
        ratio = f"{(rd + wr) / comp:.2f}" if comp else "-"
        comp_mb = f"{comp / 1e6:.1f}" if comp else "-"
        lines.append(f"| `{k}` | {f[k]:.0f} | {w.get(k, 0.0):.0f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{comp_mb} | {ratio} |")
    with open(table_path, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
    return fs, ws, lines


def _counter_rows(folder):
    """kernel -> {counter: mean value, '_ns': mean dispatch duration}."""
    acc, dur = {}, {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = _short(r["Kernel_Name"])
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            dur.setdefault(k, []).append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return {k: dict({c: sum(v) / len(v) for c, v in cs.items()}, _ns=sum(dur[k]) / len(dur[k]))
            for k, cs in acc.items()}


def _agent(folder):
    for f in glob.glob(os.path.join(folder, "**", "*agent_info.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Agent_Type"] == "GPU":
                return int(r["Num_Xcc"]), int(r["Cu_Count"]), int(r["Simd_Per_Cu"])
    return 8, 256, 4


def _trace_ns(folder):
    """kernel -> average duration (ns) from a --kernel-trace --stats run."""
    rows = csv.DictReader(open(_one(os.path.join(folder, "**", "*kernel_stats.csv"))))
    return {_short(r["Name"]): float(r["AverageNs"]) for r in rows}


HEADLINE_ARGS = "--steps 2 --warmup 1 --no-naive --no-cpu --no-extra"


def counters(mfma_dir, lds_dir, trace_dir, out, workload, bench_args=HEADLINE_ARGS):
    """Matrix-core busy cycles and bf16 MFMA operations, LDS conflicts and
    activity per kernel; bench_args are the bench.py arguments of the runs."""
    m, l = _counter_rows(mfma_dir), _counter_rows(lds_dir)
    tns = _trace_ns(trace_dir)
    xcc, cus, simds = _agent(mfma_dir)
    lines = [f"# Matrix-core and LDS counters per launch: {workload}", "",
             "Commands (from the repository root on one MI355X, after "
             "`cd /tmp && export TMPDIR=/tmp`; `$REPO` is the repository root, `$OUT` the folder "
             "that receives the profiler output):", "", "```",
             "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES "
             "GRBM_GUI_ACTIVE --output-format csv -d $OUT/pmc_mfma -o bench -- "
             f"python3 $REPO/bench.py {bench_args}",
             "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS "
             "SQ_BUSY_CU_CYCLES --output-format csv -d $OUT/pmc_lds -o bench -- "
             f"python3 $REPO/bench.py {bench_args}",
             "python -m exact_io_aware_55_amd.profiling counters $OUT/pmc_mfma $OUT/pmc_lds "
             f"$OUT/prof profiles/<this file> {workload}" + ("" if bench_args == HEADLINE_ARGS else f" '{bench_args}'"),
             "```", "",
             f"Derived columns (the GPU reports {xcc} XCDs, {cus} CUs, {simds} SIMDs per CU):",
             "- clock = GRBM_GUI_ACTIVE / XCDs / launch duration, the duration taken from the "
             "kernel-trace run (`$OUT/prof`, the command in the kernel-trace summary): counter "
             "collection lengthens each launch, so its own timestamps would understate the clock;",
             "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x CUs x SIMDs): the share "
             "of SIMD cycles at the running clock in which the matrix core was busy;",
             "- MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (a 32x32x16 bf16 MFMA is 32768 flops "
             "and counts 64);",
             "- LDS active = SQ_LDS_IDX_ACTIVE / SQ_BUSY_CU_CYCLES.", "",
             "| kernel | launch (us, traced) | clock (GHz) | MFMA busy | MFMA flops (G) | LDS bank conflicts | "
             "LDS address conflicts | LDS instructions (M) | LDS active |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k, c in m.items():
        if not c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            continue                           # no matrix-core work (copies, fills)
        grbm = c.get("GRBM_GUI_ACTIVE", 0.0) / xcc
        ns = tns.get(k, c["_ns"])
        clock = grbm / ns if ns else 0.0
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (grbm * cus * simds) if grbm else 0.0
        flops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / 1e9
        d = l.get(k, {})
        act = d.get("SQ_LDS_IDX_ACTIVE", 0.0) / d["SQ_BUSY_CU_CYCLES"] if d.get("SQ_BUSY_CU_CYCLES") else 0.0
        lines.append(f"| `{k}` | {ns / 1e3:.0f} | {clock:.2f} | {100 * busy:.1f}% | {flops:.0f} | "
                     f"{d.get('SQ_LDS_BANK_CONFLICT', float('nan')):.0f} | "
                     f"{d.get('SQ_LDS_ADDR_CONFLICT', float('nan')):.0f} | "
                     f"{d.get('SQ_INSTS_LDS', 0.0) / 1e6:.1f} | {100 * act:.0f}% |")
    if any("fp8" in k for k in m):
        lines += ["", "The flops column counts bf16 MFMA operations only: the profiler exposes no "
                  "fp8 MFMA-operation counter on this chip (its MFMA-operation counters are F16, BF16, "
                  "F32 and F64), so the fp8 kernels read 0 there; their MFMA busy is counted."]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def compulsory_bytes(B, H, N, d, causal):
    """Bytes each kernel must move at least (bf16 tensors, fp32 statistics)."""
    t = B * H * N * d * 2                       # one [B,N,H,d] bf16 tensor
    rows = B * H * N
    pad = B * H * ((N + 63) // 64 * 64) * 4     # one padded statistic
    return {
        "fwd": 4 * t + rows * 4,                # Q K V in, O and LSE out
        "bwd_preprocess": 2 * t + rows * 4 + 2 * pad,
        "bwd_dkdv": 6 * t + 2 * pad,            # Q K V dO + stats in, dK dV out
        "bwd_dq": 6 * t + rows * 4 + 2 * pad,   # Q K V dO O + LSE in, dQ + stats out
    }


def scaling(copy_fetch, copy_write, out, B, H, d, runs):
    """HBM bytes per launch of each kernel of a causal fwd + bwd step at
    several sequence lengths (``runs``: (N, fetch_dir, write_dir), N rising).
    Bytes that grow like N (O(N d) traffic) double when N doubles; traffic
    that grew like the N x N score matrix would quadruple."""
    cf, cw = _counter(copy_fetch), _counter(copy_write)
    copy = [k for k in cf if "copy" in k.lower()][0]
    gib_kib = (1 << 30) / 1024
    fs, ws = gib_kib / cf[copy], gib_kib / cw[copy]
    per = {}
    for N, fdir, wdir in runs:
        f, w = _counter(fdir), _counter(wdir)
        comp = compulsory_bytes(B, H, N, d, True)
        for stage, (prefix, _) in STAGES.items():
            names = [k for k in f if k.startswith(prefix)]
            if names:
                k = names[0]
                per.setdefault(stage, {})[N] = (k, f[k] * fs * 1024 + w.get(k, 0.0) * ws * 1024, comp[stage])
    ns = [r[0] for r in runs]
    head = [f"# HBM bytes against sequence length: B={B} H={H} d={d} causal, forward + backward", "",
            "Commands (from the repository root on one MI355X, after `cd /tmp && export TMPDIR=/tmp`; "
            "`$REPO` is the repository root, `$OUT` the folder that receives the profiler output), "
            "for each N in " + ", ".join(str(n) for n in ns) + ":", "", "```"]
    for n in ns:
        for c, tag in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            head.append(f"rocprofv3 --pmc {c} --output-format csv -d $OUT/pmc_{tag}_n{n} -o bench -- "
                        f"python3 $REPO/bench.py --B {B} --H {H} --N {n} --d {d} --causal --steps 2 "
                        "--warmup 1 --no-naive --no-cpu --no-extra")
    head += ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_copy_fetch -o copy -- "
             "python3 $REPO/bench.py --copy-calibration",
             "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_copy_write -o copy -- "
             "python3 $REPO/bench.py --copy-calibration",
             "python -m exact_io_aware_55_amd.profiling scaling $OUT/pmc_copy_fetch $OUT/pmc_copy_write "
             f"profiles/<this file> {B} {H} {d} " + " ".join(f"{n}:$OUT/pmc_fetch_n{n}:$OUT/pmc_write_n{n}"
                                                             for n in ns),
             "```", "",
             f"Counters scaled to bytes by a plain 1 GiB device copy (x{fs:.4f} fetch, x{ws:.4f} write). "
             "MB = 10^6 bytes per launch; 'x compulsory' divides by the bytes the kernel must move "
             "(inputs read once, outputs written once); 'growth' is bytes(N) / bytes(N/2).", "",
             "| kernel | " + " | ".join(f"N={n} MB (x compulsory)" for n in ns) + " | " +
             " | ".join(f"growth {ns[i]}/{ns[i - 1]}" for i in range(1, len(ns))) + " |",
             "|---|" + "---|" * (2 * len(ns) - 1)]
    lines = []
    worst = 0.0
    for stage, byn in per.items():
        k = byn[ns[0]][0]
        cells = [f"{byn[n][1] / 1e6:.1f} (x{byn[n][1] / byn[n][2]:.2f})" for n in ns]
        growth = [byn[ns[i]][1] / byn[ns[i - 1]][1] for i in range(1, len(ns))]
        worst = max(worst, *growth)
        lines.append(f"| `{k}` | " + " | ".join(cells) + " | " + " | ".join(f"{g:.3f}" for g in growth) + " |")
    tail = ["", f"Largest growth per doubling of N: {worst:.3f} (O(N d) traffic gives 2, traffic of "
            "the N x N score matrix would give 4).  At the largest N the N x N bf16 score matrix of "
            f"all heads would be {B * H * ns[-1] ** 2 * 2 / 2 ** 30:.0f} GiB."]
    with open(out, "w") as fh:
        fh.write("\n".join(head + lines + tail) + "\n")
    return worst


VALU_COUNTERS = ("SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_MFMA SQ_VALU_MFMA_COEXEC_CYCLES "
                 "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_LDS SQ_INSTS_LDS GRBM_GUI_ACTIVE")


def valu(valu_dir, trace_dir, out, workload, bench_args=HEADLINE_ARGS):
    """Vector and transcendental instructions per MFMA, co-execution of the
    vector unit with the matrix core, and wave waiting, per kernel."""
    c_all = _counter_rows(valu_dir)
    tns = _trace_ns(trace_dir)
    xcc, cus, simds = _agent(valu_dir)
    lines = [f"# Vector-instruction counters per launch: {workload}", "",
             "Commands (from the repository root on one MI355X, after "
             "`cd /tmp && export TMPDIR=/tmp`; `$REPO` is the repository root, `$OUT` the folder "
             "that receives the profiler output):", "", "```",
             f"rocprofv3 --pmc {VALU_COUNTERS} --output-format csv -d $OUT/pmc_valu -o bench -- "
             f"python3 $REPO/bench.py {bench_args}",
             f"python -m exact_io_aware_55_amd.profiling valu $OUT/pmc_valu $OUT/prof profiles/<this file> "
             f"{workload}" + ("" if bench_args == HEADLINE_ARGS else f" '{bench_args}'"), "```", "",
             "Derived columns (per launch; SQ_INSTS_VALU counts the MFMA instructions too, so vector "
             "instructions = SQ_INSTS_VALU - SQ_INSTS_MFMA; the SQ_WAVE_CYCLES and SQ_WAIT_ANY counters "
             "count in units of 4 cycles, which cancels in their ratio):",
             "- vector / MFMA, exp2 / MFMA, LDS / MFMA: instructions issued per MFMA instruction;",
             "- co-execution = SQ_VALU_MFMA_COEXEC_CYCLES / (GRBM_GUI_ACTIVE / XCDs x CUs x SIMDs): the "
             "share of SIMD cycles in which a vector instruction ran beside a busy matrix core;",
             "- waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES: the share of resident-wave cycles spent waiting "
             "(dependencies, counters, barriers).", "",
             "| kernel | launch (us, traced) | MFMA (M) | vector / MFMA | exp2 / MFMA | LDS / MFMA | "
             "co-execution | waiting |", "|---|---|---|---|---|---|---|---|"]
    for k, c in c_all.items():
        mf = c.get("SQ_INSTS_MFMA", 0.0)
        if not mf:
            continue
        grbm = c.get("GRBM_GUI_ACTIVE", 0.0) / xcc
        co = c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / (grbm * cus * simds) if grbm else 0.0
        wait = c.get("SQ_WAIT_ANY", 0.0) / c["SQ_WAVE_CYCLES"] if c.get("SQ_WAVE_CYCLES") else 0.0
        lines.append(f"| `{k}` | {tns.get(k, c['_ns']) / 1e3:.0f} | {mf / 1e6:.1f} | "
                     f"{(c['SQ_INSTS_VALU'] - mf) / mf:.2f} | {c['SQ_INSTS_VALU_TRANS_F32'] / mf:.2f} | "
                     f"{c['SQ_INSTS_LDS'] / mf:.2f} | {100 * co:.1f}% | {100 * wait:.1f}% |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


CALIB_MODES = {0: "constant operands", 1: "random operands", 2: "random + FMA + exp2 per MFMA",
               3: "random + 2 FMA + 2 exp2 per MFMA", 4: "random, A operand from LDS",
               5: "random, A from LDS + 3 FMA + exp2 per MFMA",
               6: "random, A from LDS read once per 2 MFMAs + 3 FMA + exp2 per MFMA",
               7: "random, A from LDS + 4 FMA + exp2 per 2 MFMAs"}


def calibration(rates_json, mfma_dir, out):
    """Rates of the calibration modes (bench.py --mfma-calibration) beside the
    clock and MFMA-busy counters of their launches (the last launches of each
    kernel and grid size, after the clock has settled)."""
    import collections

    rates = None
    for line in open(rates_json):
        line = line.strip()
        if line.startswith("{") and "mfma_calibration" in line:
            rates = json.loads(line)["mfma_calibration"]
    if rates is None:
        raise SystemExit(f"no calibration line in {rates_json}")
    xcc, cus, simds = _agent(mfma_dir)
    per = collections.OrderedDict()
    for f in glob.glob(os.path.join(mfma_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            d = per.setdefault(int(r["Dispatch_Id"]), {"k": _short(r["Kernel_Name"]), "grid": int(r["Grid_Size"]),
                                                       "ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    groups = collections.OrderedDict()
    for d in per.values():
        groups.setdefault((d["k"], d["grid"]), []).append(d)
    lines = ["# Matrix-core calibration (fa_calibrate_mfma)", "",
             "Commands (from the repository root on one MI355X, after "
             "`cd /tmp && export TMPDIR=/tmp`; `$REPO` is the repository root, `$OUT` the folder "
             "that receives the profiler output):", "", "```",
             "python3 $REPO/bench.py --mfma-calibration > $OUT/calibration.json",
             "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES "
             "GRBM_GUI_ACTIVE --output-format csv -d $OUT/calib_mfma -o calib -- python3 $REPO/bench.py "
             "--mfma-calibration",
             "python -m exact_io_aware_55_amd.profiling calibration $OUT/calibration.json $OUT/calib_mfma "
             "profiles/<this file>", "```", "",
             "Each wave runs eight independent chains of v_mfma_f32_32x32x16_bf16 (32768 flops each) back "
             f"to back.  Rates from HIP events over 10 launches after a settling run; the nameplate is "
             f"2516.6 TFLOP/s (256 CUs x 4096 flop/clock x 2.4 GHz).  Counters ({xcc} XCDs, {cus} CUs, "
             f"{simds} SIMDs per CU) from the last 5 launches of each kernel and grid: clock = "
             "GRBM_GUI_ACTIVE / XCDs / launch duration (the counter run's own timestamps), MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x CUs x SIMDs), executed flops = "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512.", "",
             "| run | mode | waves per SIMD | TFLOP/s | of nameplate | clock (GHz) | MFMA busy | "
             "counted / executed flops |", "|---|---|---|---|---|---|---|---|"]
    mode_kernel = {0: ("<false, 0>", None), 1: ("<true, 0>", None), 2: ("<true, 2>", None),
                   3: ("<true, 4>", None), 4: ("calib_mfma_lds_kernel<1, 0, 0, 1>", None),
                   5: ("calib_mfma_lds_kernel<1, 3, 1, 1>", None), 6: ("calib_mfma_lds_kernel<2, 3, 1, 1>", None),
                   7: ("calib_mfma_lds_kernel<1, 4, 1, 2>", None)}
    for label, r in rates.items():
        mode = {"const": 0, "random": 1, "random_valu2": 2, "random_valu4": 3, "random_lds": 4,
                "random_lds_valu4": 5, "random_lds_half_valu4": 6,
                "random_lds_valu2p5": 7}[label.rsplit("_", 1)[0]]
        waves = int(label.rsplit("_w", 1)[1])
        grid = 256 * 4 * 64 * waves
        key = [k for k in groups if mode_kernel[mode][0] in k[0] and k[1] == grid]
        clock = busy = ratio = float("nan")
        if key:
            last = groups[key[0]][-5:]
            g = sum(d["GRBM_GUI_ACTIVE"] for d in last) / xcc
            ns = sum(d["ns"] for d in last)
            clock = g / ns
            busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in last) / (g * cus * simds)
            ex = sum(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in last) * 512 / len(last)
            flops = r["tflops"] * 1e12 * r["ms"] * 1e-3
            ratio = flops / ex if ex else float("nan")
        lines.append(f"| `{label}` | {CALIB_MODES[mode]} | {waves} | {r['tflops']:.0f} | "
                     f"{100 * r['frac']:.1f}% | {clock:.2f} | {100 * busy:.1f}% | {ratio:.3f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


MERGE_ARGS = "--lse-merge"


def merge_profile(trace_dir, fetch, write, copy_fetch, copy_write, out, workload="merge_b1_h32_n16384_d128"):
    """fa_merge's kernel time (trace) and HBM bytes (FETCH_SIZE / WRITE_SIZE
    scaled by the copy calibration) against its algorithmic bytes: both O
    arrays and both LSE arrays read, one of each written."""
    shape = {p[0]: int(p[1:]) for p in workload.split("_") if p[:1] in "bhnd" and p[1:].isdigit()}
    B, H, N, d = shape["b"], shape["h"], shape["n"], shape["d"]
    algo = 3 * B * N * H * d * 2 + 3 * B * H * N * 4
    stats = [r for r in csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_stats.csv"))))
             if _short(r["Name"]).startswith(STAGES["merge"][0])]
    fs, ws, lines = traffic(fetch, write, copy_fetch, copy_write, out, workload, {"merge": algo})
    head = [f"# fa_merge (two attention results over disjoint key ranges), {workload}", "",
            "Commands (from the repository root on one MI355X, after `cd /tmp && export TMPDIR=/tmp`; "
            "`$REPO` is the repository root, `$OUT` the folder that receives the profiler output):", "",
            "```",
            f"rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof -o merge -- python3 $REPO/bench.py {MERGE_ARGS}",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o merge -- python3 $REPO/bench.py {MERGE_ARGS}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o merge -- python3 $REPO/bench.py {MERGE_ARGS}",
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_copy_fetch -o copy -- "
            "python3 $REPO/bench.py --copy-calibration",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_copy_write -o copy -- "
            "python3 $REPO/bench.py --copy-calibration",
            "python -m exact_io_aware_55_amd.profiling merge $OUT/prof $OUT/pmc_fetch $OUT/pmc_write "
            "$OUT/pmc_copy_fetch $OUT/pmc_copy_write profiles/<this file>",
            "```", "",
            f"Algorithmic bytes per launch: {algo / 1e6:.1f} MB (two bf16 O arrays and two fp32 LSE arrays "
            "read, one of each written).  Counter bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) "
            f"scaled by a plain 1 GiB copy's (x{fs:.4f} and x{ws:.4f}).", "",
            "| kernel | calls traced | average (us) | GB/s (algorithmic) | of 8 TB/s |", "|---|---|---|---|---|"]
    for r in stats:
        t = float(r["AverageNs"])
        gbps = algo / t
        head.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {t / 1e3:.1f} | {gbps:.0f} | "
                    f"{100 * gbps / 8000:.1f}% |")
    head += ["", "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB | algorithmic MB | "
             "measured / algorithmic |", "|---|---|---|---|---|---|---|"]
    with open(out, "w") as fh:
        fh.write("\n".join(head + lines) + "\n")


def main(argv):
    if len(argv) >= 5 and argv[0] == "trace":
        trace(argv[1], argv[2], argv[3], argv[4])
    elif len(argv) >= 6 and argv[0] == "counters":
        counters(argv[1], argv[2], argv[3], argv[4], argv[5], *argv[6:7])
    elif len(argv) >= 8 and argv[0] == "scaling":
        runs = []
        for spec in argv[7:]:
            n, fdir, wdir = spec.split(":")
            runs.append((int(n), fdir, wdir))
        scaling(argv[1], argv[2], argv[3], int(argv[4]), int(argv[5]), int(argv[6]), runs)
    elif len(argv) >= 5 and argv[0] == "valu":
        valu(argv[1], argv[2], argv[3], argv[4], *argv[5:6])
    elif len(argv) >= 7 and argv[0] == "merge":
        merge_profile(*argv[1:7])
    elif len(argv) >= 4 and argv[0] == "calibration":
        calibration(argv[1], argv[2], argv[3])
    elif len(argv) >= 7 and argv[0] == "traffic":
        workload = argv[6]
        shape = {p[0]: p[1:] for p in workload.split("_") if p[:1] in "bhnd" and p[1:].isdigit()}
        comp = compulsory_bytes(int(shape["b"]), int(shape["h"]), int(shape["n"]), int(shape["d"]),
                                "causal" in workload)
        fs, ws, lines = traffic(*argv[1:5], argv[5], workload, comp)
        head = [f"# HBM traffic per launch: {workload}", "",
                "Commands (from the repository root on one MI355X, after "
                "`cd /tmp && export TMPDIR=/tmp`; `$REPO` is the repository root, `$OUT` the folder "
             "that receives the profiler output):", "", "```",
                "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o bench -- "
                "python3 $REPO/bench.py --steps 2 --warmup 1 --no-naive --no-cpu --no-extra",
                "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o bench -- "
                "python3 $REPO/bench.py --steps 2 --warmup 1 --no-naive --no-cpu --no-extra",
                "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_copy_fetch -o copy -- "
                "python3 $REPO/bench.py --copy-calibration",
                "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_copy_write -o copy -- "
                "python3 $REPO/bench.py --copy-calibration",
                "python -m exact_io_aware_55_amd.profiling traffic $OUT/pmc_fetch $OUT/pmc_write "
                f"$OUT/pmc_copy_fetch $OUT/pmc_copy_write profiles/<this file> {workload}",
                "```", "",
                f"Calibration: a plain 1 GiB device copy reads FETCH_SIZE and WRITE_SIZE that scale to its "
                f"known bytes by x{fs:.4f} (fetch) and x{ws:.4f} (write); the same factors convert the "
                "kernels' counters (KiB per dispatch) to bytes.", "",
                "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB | compulsory MB | "
                "measured / compulsory |", "|---|---|---|---|---|---|---|"]
        tail = ["", "Compulsory bytes: the forward reads Q, K, V and writes O and LSE; the preprocess "
                "reads O, dO and LSE and writes both padded row statistics; dK/dV reads Q, K, V, dO and "
                "the statistics and writes dK, dV; dQ reads Q, K, V, dO, O and LSE and writes dQ and "
                "the statistics.  The N x N score matrix never reaches HBM."]
        with open(argv[5], "w") as fh:
            fh.write("\n".join(head + lines + tail) + "\n")
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
