"""Host-side logic of bench.py (no GPU): the one-GPU contract, the copy-calibrated traffic figure,
and the uniform fan-out of the ablation."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for k, c, v in rows:
            wr.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path, monkeypatch):
    """A counter that reads half the copy's bytes doubles the kernel's reading; the copy is found
    among the other launches as the one closest to the copy size; medians over dispatches."""
    copy_kib = bench.COPY_BYTES / 1024
    k = "void ssd::verify_kernel<ssd::BF16T, 4, 2, true>(ssd::VerifyArgs)"
    _counter_csv(tmp_path / "fetch.csv", [(k, "FETCH_SIZE", 100.0), (k, "FETCH_SIZE", 102.0),
                                         (k, "FETCH_SIZE", 300.0), ("copy", "FETCH_SIZE", copy_kib / 2),
                                         ("fill", "FETCH_SIZE", 5.0)])
    _counter_csv(tmp_path / "write.csv", [(k, "WRITE_SIZE", 10.0), (k, "WRITE_SIZE", 10.0),
                                         ("copy", "WRITE_SIZE", copy_kib)])
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0123456789abcdef")
    bench.summarize_traffic(str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv"), "unit_case")
    d = json.load(open(tmp_path / "profiles" / "traffic_unit_case.json"))
    assert d["kernel_hash"] == "0123456789abcdef"
    assert abs(d["fetch"]["scale"] - 2.0) < 1e-12 and d["write"]["scale"] == 1.0
    assert d["fetch"]["raw_kib_per_launch"] == 102.0 and d["fetch"]["launches"] == 3
    assert d["bytes_per_launch"] == round(102.0 * 1024 * 2 + 10.0 * 1024)


def test_uniform_fanout_splits_the_budget_evenly():
    for K, budget in [(4, 12), (4, 32), (2, 7), (8, 0)]:
        F = bench.uniform_fanout(K, budget)
        assert len(F) == K + 1 and sum(F) == budget and max(F) - min(F) <= 1
        assert F == sorted(F, reverse=True)  # the remainder goes to the smaller k


def test_cpu_baseline_runs_the_oracle_over_worker_processes():
    import bench
    import synth
    bt = synth.make_verify_batch(3, 2, 2000, synth.BF16, 0)
    cb = bench.cpu_baseline(bt, 2, 0.3, 2)
    assert cb["cores"] == 2 and cb["kind"] == "oracle" and cb["unit"] == "rows/s"
    assert cb["value"] > 0 and cb["cpu"]
    assert bench.cpu_workers(0) == max(1, min(os.cpu_count() or 1, 16))
