"""bench.py's counter bookkeeping on the CPU: rocprofv3 counter CSVs are
averaged over the scoring kernel's dispatches, scaled by the calibration copy,
and recorded with a hash of that kernel's sources."""
from __future__ import annotations

import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(folder, counter, rows):
    os.makedirs(os.path.join(folder, "host"), exist_ok=True)
    with open(os.path.join(folder, "host", "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=FIELDS)
        wr.writeheader()
        for i, (name, v) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_write_traffic_scales_and_averages(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    k = "paged_logits_kernel"
    full = "void qsa::(anonymous namespace)::paged_logits_kernel<false, 4, 1, 4, false, false>(qsa::LogitsArgs)"
    other = "topk_window_kernel<2>(qsa::TopkArgs)"
    # calibration: a 1 GiB copy reads half its bytes on FETCH_SIZE (scale 2), all on WRITE_SIZE
    write_csv(tmp_path / "cf", "FETCH_SIZE", [("copy", 524288.0), ("small", 3.0)])
    write_csv(tmp_path / "cw", "WRITE_SIZE", [("copy", 1048576.0)])
    write_csv(tmp_path / "f", "FETCH_SIZE", [(full, 100.0), (other, 7.0), (full, 300.0)])
    write_csv(tmp_path / "w", "WRITE_SIZE", [(full, 10.0), (other, 1.0), (full, 30.0)])
    dirs = [str(tmp_path / d) for d in ("f", "w", "cf", "cw")]
    bench.write_traffic("decode_verify", k, dirs, 1024)
    t = json.load(open(tmp_path / "traffic.json"))["decode_verify"]
    assert t["fetch_bytes"] == 200 * 1024 * 2
    assert t["write_bytes"] == 20 * 1024
    assert t["bytes_per_launch"] == t["fetch_bytes"] + t["write_bytes"]
    assert t["dispatches"] == 2
    assert t["kernel"].endswith("paged_logits_kernel<false, 4, 1, 4, false, false>")
    assert t["source_hash"] == bench.source_hash(k)
    assert bench.measured_traffic("decode_verify", k) == t["bytes_per_launch"]
    # another kernel's sources do not validate this entry
    assert bench.source_hash("prefill_logits_kernel") != t["source_hash"]


def test_source_hash_ignores_comments_only():
    code = "int a; // note\n/* block\n comment */\nint b;   \n\n"
    assert bench._code_only(code) == bench._code_only("int a;\nint b;") == "int a;\nint b;"
    assert bench._code_only("int a = 1;") != bench._code_only("int a = 2;")
