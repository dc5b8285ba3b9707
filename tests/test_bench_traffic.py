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


def test_write_traffic_topk_sums_its_kernels(tmp_path, monkeypatch):
    """The split selection runs two kernels per call: their per-dispatch means
    add up to the call's bytes, under the workload's ":topk" entry."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    win = "void qsa::(anonymous namespace)::topk_window_kernel<2>(qsa::TopkArgs)"
    res = "void qsa::(anonymous namespace)::topk_resolve_kernel<2>(qsa::TopkArgs)"
    score = "void qsa::(anonymous namespace)::paged_logits_kernel<0, 4, 1, 4>(qsa::LogitsArgs)"
    write_csv(tmp_path / "cf", "FETCH_SIZE", [("copy", 524288.0)])
    write_csv(tmp_path / "cw", "WRITE_SIZE", [("copy", 1048576.0)])
    write_csv(tmp_path / "f", "FETCH_SIZE", [(score, 999.0), (win, 10.0), (res, 4.0), (win, 30.0), (res, 8.0)])
    write_csv(tmp_path / "w", "WRITE_SIZE", [(score, 99.0), (win, 1.0), (res, 2.0), (win, 3.0), (res, 2.0)])
    dirs = [str(tmp_path / d) for d in ("f", "w", "cf", "cw")]
    bench.write_traffic("decode_verify", "topk", dirs, 1024)
    t = json.load(open(tmp_path / "traffic.json"))["decode_verify:topk"]
    assert t["fetch_bytes"] == (20 + 6) * 1024 * 2
    assert t["write_bytes"] == (2 + 2) * 1024
    assert t["dispatches"] == 2
    assert "topk_window_kernel<2>" in t["kernel"] and "topk_resolve_kernel<2>" in t["kernel"]
    assert bench.measured_traffic("decode_verify", "topk") == t["bytes_per_launch"]
    assert bench.measured_traffic("decode_verify", "paged_logits_kernel") is None


def test_write_mfma_busy_fraction(tmp_path, monkeypatch):
    """MFMA busy cycles over 1,024 SIMDs x one XCD's share of GRBM_GUI_ACTIVE."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    k = "prefill_logits_kernel"
    full = "void qsa::(anonymous namespace)::prefill_logits_kernel<0, false, 8>(qsa::LogitsArgs)"
    folder = tmp_path / "m"
    os.makedirs(folder / "host", exist_ok=True)
    with open(folder / "host" / "run_counter_collection.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=FIELDS)
        wr.writeheader()
        for i, (c, v) in enumerate([("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500.0), ("GRBM_GUI_ACTIVE", 8 * 1000.0),
                                    ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 300.0), ("GRBM_GUI_ACTIVE", 8 * 1000.0)]):
            wr.writerow({"Dispatch_Id": i // 2, "Kernel_Name": full, "Counter_Name": c, "Counter_Value": v})
    bench.write_mfma("prefill_chunk", k, str(folder))
    assert bench.measured_mfma_busy("prefill_chunk", k) == 0.4


def test_write_traffic_counts_only_the_fused_call(tmp_path, monkeypatch):
    """A run that times the fused scoring + selection as its value also runs the
    two-call path: only the fused call's kernels (the scorer with the candidate
    epilogue, the candidate selection) count, not both scorers summed."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    plain = "void qsa::(anonymous namespace)::paged_logits_kernel<0, 4, 1, 4, false, false, false, 128, false>(qsa::LogitsArgs)"
    cand = "void qsa::(anonymous namespace)::paged_logits_kernel<0, 4, 1, 4, false, false, false, 128, true>(qsa::LogitsArgs)"
    sel = "void qsa::(anonymous namespace)::topk_cand_kernel<16>(qsa::TopkArgs)"
    win = "void qsa::(anonymous namespace)::topk_window_kernel<2>(qsa::TopkArgs)"
    res = "void qsa::(anonymous namespace)::topk_resolve_kernel<2>(qsa::TopkArgs)"
    write_csv(tmp_path / "cf", "FETCH_SIZE", [("copy", 524288.0)])
    write_csv(tmp_path / "cw", "WRITE_SIZE", [("copy", 1048576.0)])
    rows = [(cand, 100.0), (sel, 5.0), (plain, 90.0), (win, 7.0), (res, 9.0)] * 2
    write_csv(tmp_path / "f", "FETCH_SIZE", rows)
    write_csv(tmp_path / "w", "WRITE_SIZE", rows)
    dirs = [str(tmp_path / d) for d in ("f", "w", "cf", "cw")]
    bench.write_traffic("decode_verify", "paged_logits_kernel", dirs, 1024)
    bench.write_traffic("decode_verify", "topk", dirs, 1024)
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["decode_verify"]["fetch_bytes"] == 100 * 1024 * 2
    assert t["decode_verify"]["kernel"].endswith("128, true>")
    assert t["decode_verify:topk"]["fetch_bytes"] == 5 * 1024 * 2
    assert t["decode_verify:topk"]["kernel"].endswith("topk_cand_kernel<16>")
    # without the fused call in the run, every matching kernel of the call counts
    rows2 = [(plain, 90.0), (win, 7.0), (res, 9.0)]
    write_csv(tmp_path / "f2", "FETCH_SIZE", rows2)
    write_csv(tmp_path / "w2", "WRITE_SIZE", rows2)
    dirs2 = [str(tmp_path / d) for d in ("f2", "w2", "cf", "cw")]
    bench.write_traffic("fp8_paged", "topk", dirs2, 1024)
    assert json.load(open(tmp_path / "traffic.json"))["fp8_paged:topk"]["fetch_bytes"] == 16 * 1024 * 2
