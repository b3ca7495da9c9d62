"""Host logic of the profile converter (no GPU): counter CSVs in the layout
rocprofv3 writes are turned into bytes with the copy calibration, and the
growth of bytes with the sequence length is reported per kernel."""

import csv
import json
import os

from exact_io_aware_55_amd import profiling

COPY = "void at::native::copy_kernel(int)"
FWD = "fa::fwd_bf16_kernel<128, true, false>(int)"
DKDV = "fa::bwd_dkdv_kernel<128, true, false>(int)"


def _write(folder, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        for name, value in rows:
            w.writerow([name, "X", value, 0, 1000])


def _calibration(tmp):
    # a 1 GiB copy that reads 2^19 KiB and writes 2^20 KiB: factors 2 and 1
    _write(tmp / "cf", [(COPY, 1 << 19)])
    _write(tmp / "cw", [(COPY, 1 << 20)])


def test_counter_means_per_kernel(tmp_path):
    _write(tmp_path / "a", [(FWD, 10), (FWD, 30), (DKDV, 5)])
    got = profiling._counter(str(tmp_path / "a"))
    assert got == {"fa::fwd_bf16_kernel<128, true, false>": 20.0, "fa::bwd_dkdv_kernel<128, true, false>": 5.0}


def test_scaling_bytes_and_growth(tmp_path):
    _calibration(tmp_path)
    runs = []
    for n, f in ((4096, 1), (8192, 2), (16384, 4)):
        # forward bytes double with N (O(N d)); dK/dV bytes quadruple (O(N^2))
        _write(tmp_path / f"f{n}", [(FWD, 1000 * f), (DKDV, 1000 * f * f)])
        _write(tmp_path / f"w{n}", [(FWD, 500 * f), (DKDV, 500 * f * f)])
        runs.append((n, str(tmp_path / f"f{n}"), str(tmp_path / f"w{n}")))
    out = tmp_path / "scaling.md"
    worst = profiling.scaling(str(tmp_path / "cf"), str(tmp_path / "cw"), str(out), 1, 32, 128, runs)
    assert abs(worst - 4.0) < 1e-9
    text = out.read_text()
    fwd_row = next(line for line in text.splitlines() if line.startswith("| `fa::fwd_bf16"))
    # 1000 KiB read x 2 + 500 KiB written x 1 = 2500 KiB = 2.56 MB at N = 4096
    assert "2.6 (x" in fwd_row and fwd_row.rstrip(" |").endswith("2.000 | 2.000")
    dkdv_row = next(line for line in text.splitlines() if line.startswith("| `fa::bwd_dkdv"))
    assert dkdv_row.rstrip(" |").endswith("4.000 | 4.000")


def test_traffic_table_and_json(tmp_path):
    _calibration(tmp_path)
    _write(tmp_path / "f", [(FWD, 1000)])
    _write(tmp_path / "w", [(FWD, 400)])
    out = tmp_path / "profiles" / "traffic.md"
    os.makedirs(out.parent)
    comp = profiling.compulsory_bytes(1, 1, 1024, 128, True)
    fs, ws, lines = profiling.traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                                      str(tmp_path / "cw"), str(out), "b1_h1_n1024_d128_causal_fwd_bwd",
                                      comp)
    assert abs(fs - 2.0) < 1e-9 and abs(ws - 1.0) < 1e-9
    table = json.load(open(out.parent / "traffic.json"))
    rec = table["fwd@b1_h1_n1024_d128_causal_fwd_bwd"]
    assert rec["bytes_per_launch"] == 1000 * 2 * 1024 + 400 * 1024
    assert rec["source_sha"] == profiling.source_digest(("fa_fwd.hip", "fa_common.h", "fa_schedule.hip"))
    assert len(lines) == 1 and "fwd_bf16_kernel" in lines[0]


def test_digest_sources_agree_with_bench():
    """bench.py reports a stored traffic figure only while the digest of the
    kernel's sources matches; the two files must hash the same sources."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(profiling.ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for stage, srcs in bench.KERNELS.items():
        assert tuple(profiling.STAGES[stage][1]) == tuple(srcs), stage
        assert bench.source_digest(*srcs) == profiling.source_digest(srcs)


def test_compulsory_bytes_forward():
    # Q, K, V read and O written (bf16) plus one fp32 statistic per row
    t = 4 * 4096 * 32 * 128 * 2
    assert profiling.compulsory_bytes(4, 32, 4096, 128, False)["fwd"] == 4 * t + 4 * 32 * 4096 * 4


def test_kernel_names_mangled_or_not():
    """The profiler demangles most kernel names but can leave one mangled;
    both forms map to the same short name, so a stage's kernel is found
    either way."""
    assert profiling._short("void fa::fwd_bf16_kernel<128, true, false>(int, float)") == \
        "fa::fwd_bf16_kernel<128, true, false>"
    assert profiling._short("_ZN2fa12merge_kernelILi128EEEvPKDF16bPKfS2_S4_PDF16bPfiil") == "fa::merge_kernel<128>"
    assert profiling._short("_ZN2fa15bwd_dkdv_kernelILi64ELb1ELb0EEEvPKDF16b") == \
        "fa::bwd_dkdv_kernel<64, true, false>"
    assert profiling._short("_ZN2fa12merge_kernelILi64EEEv").startswith(profiling.STAGES["merge"][0])
