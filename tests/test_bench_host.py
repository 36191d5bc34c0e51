"""Host-side logic of bench.py, run without a GPU: the one-GPU guard and the
HBM-traffic summary built from rocprofv3 counter files."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_file(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy(tmp_path):
    # a 1 GiB copy that reads FETCH_SIZE = half its bytes (KiB) and WRITE_SIZE = all of them
    kib = bench.COPY_BYTES / 1024.0
    _counter_file(tmp_path / "cf", [("copy_kernel", "FETCH_SIZE", kib / 2)])
    _counter_file(tmp_path / "cw", [("copy_kernel", "WRITE_SIZE", kib)])
    # two launches of grad_W; grad_h_reduce must not be counted as grad_h
    _counter_file(tmp_path / "kf", [("grad_W_kernel<bf16,false>", "FETCH_SIZE", 1000.0),
                                    ("grad_W_kernel<bf16,true>", "FETCH_SIZE", 3000.0),
                                    ("grad_h_reduce_kernel", "FETCH_SIZE", 99999.0)])
    _counter_file(tmp_path / "kw", [("grad_W_kernel<bf16,false>", "WRITE_SIZE", 500.0),
                                    ("grad_W_kernel<bf16,true>", "WRITE_SIZE", 500.0)])
    out = tmp_path / "traffic.json"
    rc = bench.summarize_traffic("grad_W", str(tmp_path / "kf"), str(tmp_path / "kw"), str(tmp_path / "cf"),
                                 str(tmp_path / "cw"), str(out), command="test")
    assert rc == 0
    rec = json.load(open(out))
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12 and abs(rec["write_scale"] - 1.0) < 1e-12
    assert rec["launches"] == 2
    assert abs(rec["fetch_bytes_per_launch"] - 2000.0 * 1024 * 2.0) < 1e-6
    assert abs(rec["write_bytes_per_launch"] - 500.0 * 1024) < 1e-6
    assert rec["source_hash"] == bench.kernel_source_hash()


def test_missing_counters_are_an_error(tmp_path):
    _counter_file(tmp_path / "empty", [])
    d = str(tmp_path / "empty")
    assert bench.summarize_traffic("grad_W", d, d, d, d, str(tmp_path / "x.json"), command="") == 1
    assert not os.path.exists(tmp_path / "x.json")
