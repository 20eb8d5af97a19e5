"""bench.py's rocprofv3 summary mode on small synthetic CSVs in rocprofv3's format.

The trace and counter files below are written by the test with known numbers,
so every figure the summary derives (timed-launch mean, calibration factors,
calibrated bytes, the traffic record and its kernel hash) has a hand-computed
expected value. No GPU is needed.
"""
import csv
import json
import os

import pytest

import bench

ATTN = "(anonymous namespace)::attn_fwd_bf16_d128((anonymous namespace)::MfmaArgs)"
COPY = "void at::native::copy_kernel(int*, int const*)"
FILL = "void at::native::fill_kernel(int*)"


def write_trace(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 1000
        for i, (name, dur_ns) in enumerate(rows):
            wr.writerow(["KERNEL_DISPATCH", i + 1, name, t, t + dur_ns])
            t += dur_ns + 500


def write_counters(path, rows):
    """rows: (dispatch, kernel, counter, value); one counter may repeat per dispatch."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, k, c, v in rows:
            wr.writerow([d, d, k, c, f"{v:.6f}"])


def test_short_kernel_names():
    assert bench._short_name(ATTN) == "attn_fwd_bf16_d128"
    assert bench._short_name("(anonymous namespace)::rope_kernel<__bf16, 128>(int const*, long)") == \
        "rope_kernel<__bf16, 128>"


def test_profile_summary_figures(tmp_path, monkeypatch, capsys):
    root = tmp_path / "prof"
    wl = 0   # the tiny workload: layout built on the host only
    # 3 warm-up launches of 50 us, then 10 timed launches of 100..190 us
    durs = [50_000] * bench.TRACE_WARMUP + [100_000 + 10_000 * i for i in range(bench.TRACE_STEPS)]
    write_trace(str(root / f"wl{wl}_trace" / "host" / "trace_kernel_trace.csv"),
                [(ATTN, d) for d in durs] + [("(anonymous namespace)::positions_kernel(int)", 2_000)])
    # FETCH_SIZE is reported in two rows per dispatch (summed), WRITE_SIZE in one
    write_counters(str(root / f"wl{wl}_fetch" / "host" / "pmc_counter_collection.csv"),
                   [(1, ATTN, "FETCH_SIZE", 100.0), (1, ATTN, "FETCH_SIZE", 50.0),
                    (2, ATTN, "FETCH_SIZE", 200.0), (2, ATTN, "FETCH_SIZE", 100.0),
                    (3, ATTN, "FETCH_SIZE", 90.0), (3, ATTN, "FETCH_SIZE", 60.0)])
    write_counters(str(root / f"wl{wl}_write" / "host" / "pmc_counter_collection.csv"),
                   [(1, ATTN, "WRITE_SIZE", 40.0), (2, ATTN, "WRITE_SIZE", 40.0), (3, ATTN, "WRITE_SIZE", 80.0)])
    copy_kib = bench.COPY_BYTES / 1024
    # the calibration run: a fill of the source, then the copy launched twice
    write_counters(str(root / "copy_fetch" / "host" / "pmc_counter_collection.csv"),
                   [(1, FILL, "FETCH_SIZE", 10.0), (2, COPY, "FETCH_SIZE", copy_kib / 2),
                    (3, COPY, "FETCH_SIZE", copy_kib / 2)])
    write_counters(str(root / "copy_write" / "host" / "pmc_counter_collection.csv"),
                   [(1, FILL, "WRITE_SIZE", copy_kib), (2, COPY, "WRITE_SIZE", copy_kib),
                    (3, COPY, "WRITE_SIZE", copy_kib)])
    write_counters(str(root / f"wl{wl}_sq" / "host" / "pmc_counter_collection.csv"),
                   [(1, ATTN, "GRBM_GUI_ACTIVE", 8.0e6), (1, ATTN, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5e6 * 1024)])
    traffic = tmp_path / "attn_traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))

    assert bench.main(["--profile-summary", "--workload", str(wl), "--profile-dir", str(root),
                       "--record-traffic"]) == 0
    out = capsys.readouterr().out
    # timed launches: mean of 100..190 us = 145 us, median 145 us
    assert "mean 145.0 us, median 145.0 us" in out
    assert f"{bench.TRACE_WARMUP} warm-up + {bench.TRACE_STEPS} timed steps" in out
    # calibration: the copy's FETCH_SIZE is half its bytes, WRITE_SIZE all of them
    assert "FETCH_SIZE x 1024 x 2.000 and WRITE_SIZE x 1024 x 1.000" in out
    # attention: median FETCH 150 KiB (of 150, 300, 150), median WRITE 40 KiB
    expect = int(round((150.0 * 2 + 40.0) * 1024))
    rec = json.loads(traffic.read_text())["tiny-fp32"]
    assert rec["hbm_bytes_per_launch"] == expect
    assert rec["kernel_hash"] == bench.kernel_source_hash()
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    # MFMA busy: 0.5e6 * 1024 busy cycles / (8e6 / 8 XCDs * 1024 SIMDs) = 50 %
    assert "MFMA busy 50.0 %" in out
    # every command of the recipe is quoted in the summary
    for _, _, cmd in bench.profile_recipe(wl, str(root)):
        if "--pmc TCC" not in cmd:
            assert cmd in out


def test_profile_recipe_names_committed_programs_only():
    for _, out, cmd in bench.profile_recipe(2, "rocprof_out"):
        assert out.startswith("rocprof_out/")
        assert "-- python3 bench.py" in cmd
        assert cmd.startswith("timeout -s KILL ")
        assert "cd " not in cmd


def test_profile_summary_requires_the_runs(tmp_path):
    with pytest.raises(SystemExit):
        bench.main(["--profile-summary", "--workload", "0", "--profile-dir", str(tmp_path)])
