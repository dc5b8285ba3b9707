"""Benchmark: one paged MQA-logits + top-k call per step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_verify]

Prints one JSON line.  The default workload is the decode-verify batch
(9 requests x 4 MTP rows, 4 index heads, D = 128, bf16, contexts uniform in
16,000..32,000 compressed columns, block 16, top-k 2048).  Inputs are seeded and
synthetic and already resident in HBM when timing starts; the step cycles
through enough input replicas that no step finds its keys in L2 or the 256 MB
Infinity Cache (each replica's bytes are read again only after more than
512 MB of other traffic).

``value`` is microseconds per call (scoring + selection): HIP events around the
K timed steps, nothing else in between.  ``roofline`` covers the scoring kernel:
algorithmic bytes per launch / the mean duration of its launches, from a second
pass over the same K steps in which every kernel dispatch records a start and an
end HIP event itself (on the stream the kernels run on), against the MI355X HBM
peak of 8 TB/s.  ``cpu_baseline`` is
the CPU oracle timed on this host's cores on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per paged MQA-logits+top-k call; achieved HBM GB/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "paged_mqa_logits_block_amd", "csrc")
# each scoring kernel's own source file; the planner and the shared headers
# are part of every kernel's hash
KERNEL_FILES = {"paged_logits_kernel": "logits_decode.hip", "looped_logits_kernel": "logits_looped.hip",
                "mtp_fp8_kernel": "logits_mtp.hip", "prefill_logits_kernel": "logits_prefill.hip"}
COMMON_SOURCES = ("logits.hip", "logits_frag.h", "qsa_device.h", "qsa_internal.h")

DESCRIPTIONS = {
    "tiny": "2 requests x 4 rows, 4 heads, D=128, bf16, ctx 1000/3000, block 16, top-k 256",
    "decode_verify": "9 requests x 4 MTP rows (36 rows), 4 heads, D=128, bf16 q/k N(0,1), "
                     "ctx U[16000,32000] compressed columns, block 16, top-k 2048",
    "single_row_mixed": "64 requests x 1 row, 4 heads zero-padded to 16, D=128, bf16, "
                        "ctx log-uniform 5000..65600, width 65600, block 64, top-k 2048",
    "fp8_paged": "16 requests x 4 rows, 64 heads, D=128, fp8 e4m3 q/k, per-key f32 scale, "
                 "w U(0,1), kv_len 32768, co-packed KVB=64, top-k 2048",
    "prefill_chunk": "1 request, 16384 rows at positions 98304..114687, 4 heads, D=128, bf16, "
                     "ctx (pos+1)//4, block 64, top-k 2048",
    "decode_verify_fp16": "decode_verify with fp16 q/k: 9 requests x 4 MTP rows, 4 heads, D=128, "
                          "ctx U[16000,32000], block 16, top-k 2048",
    "prefill_chunk_fp16": "prefill_chunk with fp16 q/k: 1 request, 16384 rows, 4 heads, D=128, "
                          "ctx (pos+1)//4, block 64, top-k 2048",
    "fp8_paged_kvb1": "fp8_paged with one key per block (per-token co-packed layout, 132 B blocks): "
                      "16 requests x 4 rows, 64 heads, fp8, kv_len 32768, top-k 2048",
    "fp8_paged_shuffled": "fp8_paged with the keys of each co-packed KVB=64 block preshuffled in "
                          "16x16-byte tiles: 16 requests x 4 rows, 64 heads, kv_len 32768, top-k 2048",
    "decode_verify_d64": "decode_verify with head dim 64: 9 requests x 4 MTP rows, 4 heads, D=64, bf16, "
                         "ctx U[16000,32000], block 16, top-k 2048",
}


def algorithmic_bytes(inp):
    """Bytes the scoring must move at least once: keys (and scales) once per
    request, q, w, the table entries used, ctx / row_to_req, and every output
    column (-inf included)."""
    import numpy as np
    B = inp.block_size
    kv = np.zeros(inp.num_reqs, dtype=np.int64)
    ce = inp.ctx_eff()
    for r in range(inp.num_rows):
        kv[inp.row_to_req[r]] = max(kv[inp.row_to_req[r]], int(ce[r]))
    key_b = inp.key_bytes_per_col()
    qb = inp.q.nbytes + (0 if inp.w is None else inp.w.nbytes)
    table = int(np.sum((kv + B - 1) // B)) * 4
    reads = int(np.sum(kv)) * key_b + qb + table + 8 * inp.num_rows
    writes = inp.num_rows * inp.width * 4
    return reads, writes


def scoring_kernel(inp):
    """The scoring kernel the library picks for this shape (the same rule as
    its planner): the prefill variant for bf16 or fp16, 4 heads and one request with
    256+ rows and blocks of a multiple of 32 columns; the 4-row variant for fp8
    with 32/64 heads and 4 rows per request; the looped variant for other fp8
    shapes with 16+ heads and blocks of a multiple of 16 columns; the per-tile
    variant otherwise."""
    if inp.head_dim != 128:
        return "paged_logits_kernel"
    if (inp.dtype in ("bf16", "fp16") and inp.num_heads == 4 and inp.num_reqs == 1 and inp.num_rows >= 256
            and inp.block_size % 32 == 0):
        return "prefill_logits_kernel"
    if inp.dtype == "fp8" and inp.num_heads in (32, 64) and inp.num_rows == 4 * inp.num_reqs:
        return "mtp_fp8_kernel"
    if inp.dtype == "fp8" and inp.num_heads >= 16 and inp.block_size % 16 == 0:
        return "looped_logits_kernel"
    return "paged_logits_kernel"


def _code_only(text):
    """Source text without comments, trailing blanks and blank lines: edits to
    comments do not change what the counters measured."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def source_hash(kernel):
    """Hash of the code (comments stripped) a scoring kernel is built from."""
    h = hashlib.sha256()
    for f in (KERNEL_FILES[kernel], *COMMON_SOURCES):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    once the kernel's sources differ from the ones the counters were taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("source_hash") != source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


def _counter_rows(folder, counter):
    """(kernel name, value) per dispatch from rocprofv3 counter-collection CSVs
    under `folder`."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r.get("Kernel_Name", ""), float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {folder}")
    return rows


def write_traffic(workload, kernel, dirs, calib_mib):
    """Record the scoring kernel's HBM bytes per launch in profiles/traffic.json.

    dirs = (FETCH_SIZE run, WRITE_SIZE run, FETCH_SIZE run of the calibration
    copy, WRITE_SIZE run of the calibration copy): rocprofv3 output folders.
    Both counters read KiB per dispatch; each is scaled by what it reads for a
    plain device copy of calib_mib MiB each way (the copy's largest dispatch)."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    copy_kib = calib_mib * 1024.0
    out = {}
    for name, d, cd in (("fetch", fetch_dir, cfetch_dir), ("write", write_dir, cwrite_dir)):
        counter = "FETCH_SIZE" if name == "fetch" else "WRITE_SIZE"
        scale = copy_kib / max(v for _, v in _counter_rows(cd, counter))
        vals = [(k, v) for k, v in _counter_rows(d, counter) if kernel in k]
        if not vals:
            raise SystemExit(f"no {kernel} dispatches with {counter} under {d}")
        out[name] = (statistics.mean(v for _, v in vals) * 1024.0 * scale, scale, len(vals), vals[0][0])
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    full_name = out["fetch"][3].removeprefix("void ")
    table[workload] = {
        "source_hash": source_hash(kernel),
        "kernel": full_name[:full_name.rindex("(")] if full_name.endswith(")") else full_name,
        "fetch_bytes": round(out["fetch"][0]),
        "write_bytes": round(out["write"][0]),
        "bytes_per_launch": round(out["fetch"][0] + out["write"][0]),
        "fetch_scale": round(out["fetch"][1], 4),
        "write_scale": round(out["write"][1], 4),
        "dispatches": out["fetch"][2],
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({workload: table[workload]}))


def cpu_baseline(inp, budget_s=20.0):
    import numpy as np
    import oracle
    threads = oracle.max_threads()
    # time one call on a row sample that keeps the run within the budget
    rows = list(range(inp.num_rows))
    t0 = time.perf_counter()
    oracle.paged_logits(inp, rows=rows[:1])
    one = max(time.perf_counter() - t0, 1e-4)
    n = max(1, min(inp.num_rows, int(budget_s / 3 / one)))
    n -= n % max(1, min(n, 4))
    sample = rows[:max(n, 1)]
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        lg = oracle.paged_logits(inp, rows=sample)
        oracle.topk(lg.astype(np.float32), inp.ctx_lens[sample], inp.topk)
        times.append(time.perf_counter() - t0)
    per_call_us = statistics.median(times) * 1e6 * inp.num_rows / len(sample)
    return {"value": round(per_call_us, 1), "unit": "µs/call", "cores": threads, "kind": "oracle",
            "sample": f"{len(sample)} of {inp.num_rows} rows, scoring + top-k, median of 3, "
                      f"scaled by rows; float64 C loops, OpenMP over rows"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_verify", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CALIB_FETCH_DIR",
                                                          "CALIB_WRITE_DIR"),
                    help="record the scoring kernel's counter bytes from rocprofv3 --pmc output "
                         "folders (FETCH_SIZE, WRITE_SIZE, and both for a --calib-copy-mib run); "
                         "no GPU needed")
    ap.add_argument("--calib-mib", type=int, default=1024, help="size of the calibration copy")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the scoring path has no multi-GPU variant in this library)", file=sys.stderr)
        sys.exit(2)

    if args.write_traffic:
        import qsa_inputs
        inp = qsa_inputs.make_config(args.workload)
        write_traffic(args.workload, scoring_kernel(inp), args.write_traffic, args.calib_mib)
        return

    import numpy as np
    import torch

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_each_way": n * 4}))
        return

    import paged_mqa_logits_block_amd as qsa
    import qsa_inputs
    from qsa_inputs.device import to_device

    inp = qsa_inputs.make_config(args.workload)
    reads, writes = algorithmic_bytes(inp)
    per_call = reads + writes
    reps = max(1, min(16, math.ceil(600e6 / max(inp.kcache.nbytes + writes, 1))))
    devs = [to_device(inp) for _ in range(reps)]
    outs = [torch.empty((inp.num_rows, inp.width), dtype=torch.float32, device="cuda") for _ in range(reps)]
    idx = torch.empty((inp.num_rows, inp.topk), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    # calls validated once per replica; a step only crosses the C ABI twice
    calls = []
    for d, o in zip(devs, outs):
        calls.append((qsa.PreparedLogits(d.q, d.kcache, d.block_table, d.ctx_lens, d.row_to_req, o,
                                         width=d.width, block_size=d.block_size, w=d.w,
                                         kscale=d.kscale, layout=d.layout, stream=stream),
                      qsa.PreparedTopk(o, d.ctx_lens, d.topk, idx, stream=stream)))

    def step(i, evs=None):
        lg, tk = calls[i % reps]
        if evs is None:
            lg()
            tk()
        else:
            lg((evs[0], evs[1]))
            tk((evs[2], evs[3]))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps, events only around the whole region
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    us_per_call = total_ms * 1e3 / args.steps

    # kernel durations: the same K steps again, each kernel timed by HIP events
    # that its own dispatch records at kernel start and end (on the stream the
    # kernels run on); these events add host and GPU time per launch, so they
    # stay out of the region above
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e4 in evs:
        for e in e4:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    logit_us = statistics.mean(e[0].elapsed_time(e[1]) for e in evs) * 1e3
    topk_us = statistics.mean(e[2].elapsed_time(e[3]) for e in evs) * 1e3

    achieved = per_call / (logit_us * 1e-6) / 1e9
    traffic = measured_traffic(args.workload, scoring_kernel(inp))
    line = {
        "metric": METRIC,
        "value": round(us_per_call, 2),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic (seeded generators; shapes of the pages' workloads)",
        "config": {"workload": args.workload, "description": DESCRIPTIONS[args.workload],
                   "rows": inp.num_rows, "width": inp.width, "heads": inp.num_heads,
                   "block": inp.block_size, "topk": inp.topk, "input_replicas": reps},
        "logits_us": round(logit_us, 2),
        "topk_us": round(topk_us, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": scoring_kernel(inp), "algorithmic_bytes": per_call,
                     "algorithmic_read_bytes": reads, "algorithmic_write_bytes": writes},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
