"""Host logic of bench.py (no GPU): the one-GPU contract, the pair count the
flop figures use, the traffic record's source check and the counter summary."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr


def test_pair_count_is_state_pairs_plus_causal_frame_pairs():
    # T queries over `kept` state keys, plus the frame's own keys causally.
    T, kept = 5, 7
    brute = sum(kept + i + 1 for i in range(T))
    assert bench.pair_count(T, kept) == brute
    assert bench.pair_count(256, 4096) == 1_081_472


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"source_sha256": bench.kernel_source_hash(), "bytes_per_launch": 1234.5}
    (prof / "attn_fwd_w_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("attn_fwd", "w") == 1234.5
    rec["source_sha256"] = "0" * 64   # counters taken on another kernel source
    (prof / "attn_fwd_w_traffic.json").write_text(json.dumps(rec))
    assert bench.load_traffic("attn_fwd", "w") is None
    assert bench.load_traffic("attn_fwd", "absent") is None


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, grid, value in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                        "Counter_Value": value})


def test_counter_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    mib = 256
    copy_bytes = mib * (1 << 20)
    # The copy's FETCH_SIZE reads half its bytes (scale x2), WRITE_SIZE all of them (x1);
    # values are KiB per dispatch.  Three attn_fwd dispatches: the median is taken.
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1024, copy_bytes / 2 / 1024),
                                       ("__amd_rocclr_copyBuffer", 16, 1.0),
                                       ("void attn_fwd_kernel<...>", 1, 100.0),
                                       ("void attn_fwd_kernel<...>", 1, 300.0),
                                       ("void attn_fwd_kernel<...>", 1, 200.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1024, copy_bytes / 1024),
                                       ("void attn_fwd_kernel<...>", 1, 50.0)])
    rec = bench.summarize_pmc(str(fetch), str(write), "w", mib)
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2 + 50.0 * 1024)
    assert rec["source_sha256"] == bench.kernel_source_hash()
    assert json.loads((tmp_path / "profiles" / "attn_fwd_w_traffic.json").read_text()) == rec
