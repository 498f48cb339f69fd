"""bench.py's host-side contract, on the CPU: one GPU only (--gpus N > 1 exits with a message
before touching a GPU), argument checks, and the rocprofv3 summary that the profiles and the
traffic records come from (averages over the chosen dispatches, counters scaled by a plain
copy's reading)."""
import csv
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    res = _run("--gpus", "2")
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_steps_must_be_positive():
    res = _run("--steps", "0")
    assert res.returncode != 0 and "--steps" in res.stderr


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_profile_summary_averages_and_scales(tmp_path):
    kern = "my_kernel(int)"
    # 8 dispatches of the kernel (durations 10, 20, ..., 80 us), one of another kernel
    trace = [[kern, d, 1000 * d * 1000, 1000 * d * 1000 + 10000 * (d + 1)] for d in range(8)]
    trace.append(["other_kernel()", 99, 0, 5000])
    _write(str(tmp_path / "tr" / "run_kernel_trace.csv"), ["Kernel_Name", "Dispatch_Id", "Start_Timestamp",
                                                           "End_Timestamp"], trace)
    _write(str(tmp_path / "tr" / "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
           [[kern, 8, 45000, 10000, 80000]])
    # counters: FETCH_SIZE 100*(d+1) KiB, WRITE_SIZE 50 KiB per dispatch; a 256 MiB copy reads as
    # 131072 KiB fetched (scale x2) and 262144 KiB written (scale x1)
    _write(str(tmp_path / "pmc_FETCH_SIZE" / "run_counter_collection.csv"),
           ["Kernel_Name", "Dispatch_Id", "Counter_Value"], [[kern, d, 100 * (d + 1)] for d in range(8)])
    _write(str(tmp_path / "pmc_WRITE_SIZE" / "run_counter_collection.csv"),
           ["Kernel_Name", "Dispatch_Id", "Counter_Value"], [[kern, d, 50] for d in range(8)])
    _write(str(tmp_path / "copy_FETCH_SIZE" / "run_counter_collection.csv"),
           ["Kernel_Name", "Dispatch_Id", "Counter_Value"], [["copy", d, 131072] for d in range(5)])
    _write(str(tmp_path / "copy_WRITE_SIZE" / "run_counter_collection.csv"),
           ["Kernel_Name", "Dispatch_Id", "Counter_Value"], [["copy", d, 262144] for d in range(5)])
    res = _run("--summarize-profile", "--trace-dir", str(tmp_path / "tr"), "--kernel", "my_kernel",
               "--skip", "2", "--last", "3", "--pmc-dir", str(tmp_path / "pmc"), "--copy-dir", str(tmp_path / "copy"),
               "--pmc-skip", "4", "--pmc-last", "2")
    assert res.returncode == 0, res.stderr
    out = res.stdout
    # dispatches 2..4: 30, 40, 50 us
    assert "dispatches 2..4 of the kernel): average 40.00 us, median 40.00 us" in out
    # FETCH over dispatches 4, 5: 500 and 600 KiB -> 550 KiB, x2 -> 1100 KiB = 1.13 MB
    assert "FETCH_SIZE: 550.0 KiB per dispatch over 2 timed dispatches" in out and "scale x2.000" in out
    fetch_mb = 550 * 2 * 1024 / 1e6
    assert f"-> {fetch_mb:.2f} MB per launch" in out
    write_mb = 50 * 1 * 1024 / 1e6
    assert f"(scaled FETCH + WRITE): {fetch_mb + write_mb:.2f} MB" in out
    assert "other_kernel" not in out
    assert np.isclose(fetch_mb + write_mb, 1.1776)


def test_traffic_record_is_used_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "KERNEL_SRC", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    import json
    rec.write_text(json.dumps({"k": {"bytes_per_launch": 123.0, "source_sha256": bench._sha256(str(src))}}))
    assert bench.recorded_traffic("k", "k.hip") == 123.0
    assert bench.recorded_traffic("missing", "k.hip") is None
    src.write_text("kernel v2\n")                       # any edit voids the record
    assert bench.recorded_traffic("k", "k.hip") is None
    # every committed record matches its kernel source as it stands
    committed = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    csrc = os.path.join(ROOT, "hierarchical_kv_cache_hs_amd", "csrc")
    shas = {bench._sha256(os.path.join(csrc, f)) for f in os.listdir(csrc) if f.endswith(".hip")}
    for key, r in committed.items():
        assert r["source_sha256"] in shas, f"{key}: traffic record of a kernel source that has changed"
