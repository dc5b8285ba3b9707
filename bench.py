"""Benchmark: one paged MQA-logits + top-k call per step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_chunk]

Prints one JSON line.  The default workload is the largest of the five
single-GPU configurations, the prefill chunk (1 request, 16,384 query rows at
positions 98,304..114,687, 4 index heads, D = 128, bf16, causal visibility
(pos + 1) // 4 columns, block 64, top-k 2048).  Inputs are seeded and synthetic
and already resident in HBM when timing starts; the step cycles through enough
input replicas that no step finds its keys in L2 or the 256 MB Infinity Cache
(each replica's bytes are read again only after more than 512 MB of other
traffic), except where one replica alone is larger than that.

``value`` is microseconds per call of the library's full call,
qsa_paged_logits_topk (the logits written, then the top-k of them; on decode
shapes the scoring epilogue feeds the selection): HIP events around the K timed
steps, nothing else in between.  ``two_call_value`` times the same work as two
calls (qsa_paged_logits, then qsa_topk).  ``roofline`` has one entry per kernel
of the call (``kernels``: scoring, then selection) and repeats the dominant
one's figures at its top level: algorithmic bytes per launch / the mean duration
of its launches, from a third pass over the same K steps in which every kernel
dispatch records a start and an end HIP event itself (on the stream the kernels
run on), against the MI355X HBM peak of 8 TB/s; the scorer also reports its MFMA
rate against the dense peak of its dtype.  ``configs`` summarises the same
figures for all five workloads (shorter runs).  ``cpu_baseline`` is the CPU
oracle timed on this host's cores on a row sample of the headline workload.
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
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp8": 5000.0}
SIMDS = 1024  # 256 CUs x 4
XCDS = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "paged_mqa_logits_block_amd", "csrc")
# each scoring kernel's own source file; the planner and the shared headers
# are part of every kernel's hash
KERNEL_FILES = {"paged_logits_kernel": "logits_decode.hip", "looped_logits_kernel": "logits_looped.hip",
                "mtp_fp8_kernel": "logits_mtp.hip", "prefill_logits_kernel": "logits_prefill.hip",
                "topk": "topk.hip"}
COMMON_SOURCES = ("logits.hip", "logits_frag.h", "qsa_device.h", "qsa_internal.h")
TOPK_COMMON_SOURCES = ("qsa_device.h", "qsa_internal.h")
# the top-k launch rule of the library's planner: rows shared by several
# workgroups (with a workspace) for at most 128 rows wider than 4096 columns,
# unless 48 or more rows fit the register path (32,768 columns)
TOPK_SPLIT_MAX_ROWS = 128
TOPK_SPLIT_MIN_WIDTH = 4097
TOPK_ROWS_MIN_ROWS = 48
TOPK_REGISTER_WIDTH = 32768

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
    "fp8_paged_ragged": "fp8_paged with 1..8 verify rows per request (63 rows over 16 requests): 64 heads, fp8, "
                        "w U(0,1), kv_len 32768, co-packed KVB=64, top-k 2048",
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
    with 32/64 heads and 2+ rows per request on average; the looped variant for other fp8
    shapes with 16+ heads and blocks of a multiple of 16 columns; the per-tile
    variant otherwise."""
    if inp.head_dim != 128:
        return "paged_logits_kernel"
    if (inp.dtype in ("bf16", "fp16") and inp.num_heads == 4 and inp.num_reqs == 1 and inp.num_rows >= 256
            and inp.block_size % 32 == 0):
        return "prefill_logits_kernel"
    if (inp.dtype == "fp8" and inp.num_heads in (32, 64) and inp.num_rows >= 2 * inp.num_reqs
            and (inp.layout != "copacked_shuffled" or inp.block_size % 64 == 0)):
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
    """Hash of the code (comments stripped) a kernel is built from: a scoring
    kernel's own file plus the planner and shared headers, or the top-k file
    ("topk") plus the shared headers."""
    common = TOPK_COMMON_SOURCES if kernel == "topk" else COMMON_SOURCES
    h = hashlib.sha256()
    for f in (KERNEL_FILES[kernel], *common):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _traffic_key(workload, kernel):
    """Entry of profiles/traffic.json: the workload's name for its scoring
    kernel, "<workload>:topk" for its top-k kernels."""
    return f"{workload}:topk" if kernel == "topk" else workload


def _traffic_entry(workload, kernel):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(_traffic_key(workload, kernel))
    if not e or e.get("source_hash") != source_hash(kernel):
        return None
    return e


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    once the kernel's sources differ from the ones the counters were taken on."""
    e = _traffic_entry(workload, kernel)
    return None if e is None else e.get("bytes_per_launch")


def measured_mfma_busy(workload, kernel):
    """Fraction of SIMD cycles the MFMA unit was busy during the scoring kernel,
    from a committed rocprofv3 counter run (SQ_VALU_MFMA_BUSY_CYCLES over
    1,024 SIMDs x the kernel's GRBM_GUI_ACTIVE cycles per XCD), or None."""
    e = _traffic_entry(workload, kernel)
    return None if e is None else e.get("mfma_busy_frac")


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


def _matches(kernel, name):
    """Whether a dispatch's kernel name belongs to `kernel` ("topk": any of the
    top-k kernels)."""
    base = name.removeprefix("void ")
    if base.endswith(")"):  # the argument list
        base = base[:base.rindex("(")]
    if "<" in base:  # template arguments
        base = base[:base.index("<")]
    base = base.split("::")[-1]
    return base.startswith("topk_") if kernel == "topk" else base.startswith(kernel)


def _template_args(name):
    """The template argument list of a dispatch's kernel name, as strings."""
    base = name.removeprefix("void ")
    if base.endswith(")"):
        base = base[:base.rindex("(")]
    if "<" not in base:
        return []
    return [a.strip() for a in base[base.index("<") + 1:base.rindex(">")].split(",")]


def _value_path(kernel, names):
    """The kernels of the call that `value` times, among the dispatched names:
    a run that also timed the fused scoring + selection (topk_cand_kernel
    dispatched) times it as `value`, so only its kernels count -- the per-tile
    scorer with the candidate epilogue (last template argument true) and the
    candidate selection; the two-call path's kernels of the same run do not."""
    fused = any(_matches("topk_cand_kernel", n) for n in names)
    if not fused:
        return set(names)
    keep = set()
    for n in names:
        if kernel == "topk":
            if _matches("topk_cand_kernel", n):
                keep.add(n)
        elif not _matches("paged_logits_kernel", n) or _template_args(n)[-1:] == ["true"]:
            keep.add(n)
    return keep


def _per_call(kernel, rows):
    """Mean counter value per call: the mean over each matching kernel's
    dispatches, summed over the kernels of a call (the split top-k runs two);
    with the fused call in the run, only its kernels."""
    by = {}
    for k, v in rows:
        if _matches(kernel, k):
            by.setdefault(k, []).append(v)
    names = _value_path(kernel, [k for k, _ in rows])
    by = {k: v for k, v in by.items() if k in names}
    if not by:
        return None, 0, ""
    return (sum(statistics.mean(v) for v in by.values()), min(len(v) for v in by.values()),
            " + ".join(sorted(by)))


def _load_table():
    try:
        with open(TRAFFIC_FILE) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def _save_table(table):
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")


def _short_name(full):
    names = []
    for n in full.split(" + "):
        n = n.removeprefix("void ")
        names.append(n[:n.rindex("(")] if n.endswith(")") else n)
    return " + ".join(names)


def write_traffic(workload, kernel, dirs, calib_mib):
    """Record a kernel's HBM bytes per call in profiles/traffic.json.

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
        mean, n, full = _per_call(kernel, _counter_rows(d, counter))
        if mean is None:
            raise SystemExit(f"no {kernel} dispatches with {counter} under {d}")
        out[name] = (mean * 1024.0 * scale, scale, n, full)
    table = _load_table()
    key = _traffic_key(workload, kernel)
    entry = table.get(key, {})
    if entry.get("source_hash") != source_hash(kernel):
        entry = {}
    entry.update({
        "source_hash": source_hash(kernel),
        "kernel": _short_name(out["fetch"][3]),
        "fetch_bytes": round(out["fetch"][0]),
        "write_bytes": round(out["write"][0]),
        "bytes_per_launch": round(out["fetch"][0] + out["write"][0]),
        "fetch_scale": round(out["fetch"][1], 4),
        "write_scale": round(out["write"][1], 4),
        "dispatches": out["fetch"][2],
    })
    table[key] = entry
    _save_table(table)
    print(json.dumps({key: entry}))


def write_mfma(workload, kernel, folder):
    """Record the scoring kernel's MFMA busy fraction from a rocprofv3 run with
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (GRBM_GUI_ACTIVE is summed over
    the 8 XCDs, so one XCD's cycles are a eighth of it)."""
    busy, n, full = _per_call(kernel, _counter_rows(folder, "SQ_VALU_MFMA_BUSY_CYCLES"))
    gui, _, _ = _per_call(kernel, _counter_rows(folder, "GRBM_GUI_ACTIVE"))
    if busy is None or gui is None:
        raise SystemExit(f"no {kernel} dispatches with the MFMA counters under {folder}")
    frac = busy / (SIMDS * gui / XCDS)
    table = _load_table()
    key = _traffic_key(workload, kernel)
    entry = table.get(key, {})
    if entry.get("source_hash") != source_hash(kernel):
        entry = {"source_hash": source_hash(kernel), "kernel": _short_name(full)}
    entry.update({"mfma_busy_frac": round(frac, 4), "mfma_busy_cycles": round(busy),
                  "gui_active_cycles": round(gui), "mfma_dispatches": n})
    table[key] = entry
    _save_table(table)
    print(json.dumps({key: entry}))


def topk_plan(inp):
    """Which top-k kernels the library runs for this shape with its automatic
    workspace: "split" (window + resolve kernels) or "rows" (one kernel)."""
    r, w = inp.num_rows, inp.width
    if r <= TOPK_SPLIT_MAX_ROWS and w >= TOPK_SPLIT_MIN_WIDTH and not (r >= TOPK_ROWS_MIN_ROWS and w <= TOPK_REGISTER_WIDTH):
        return "split"
    return "rows"


def topk_bytes(inp):
    """Bytes the selection must move at least once: every visible logit read
    (sum of the rows' visible counts, 4 B each), the visible counts, and the
    k indices written per row."""
    import numpy as np
    n = np.clip(inp.ctx_lens.astype(np.int64), 0, inp.width)
    reads = int(np.sum(n)) * 4 + 4 * inp.num_rows
    writes = inp.num_rows * inp.topk * 4
    return reads, writes


def scoring_flops(inp):
    """2 H D per visible (row, column): the q.k contraction of every head."""
    import numpy as np
    return 2 * inp.num_heads * inp.head_dim * int(np.sum(inp.ctx_eff()))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(inp, budget_s=15.0):
    """The oracle (scoring + top-k) on a sample of the workload's first rows,
    sized so that three timed runs take about budget_s seconds of wall time."""
    import numpy as np
    import oracle
    threads = oracle.max_threads()
    rows = list(range(inp.num_rows))
    # calibrate on a trial large enough to occupy every thread
    trial = rows[:min(inp.num_rows, max(4, 2 * threads))]
    t0 = time.perf_counter()
    oracle.paged_logits(inp, rows=trial)
    per_row = max(time.perf_counter() - t0, 1e-4) / len(trial)
    n = max(1, min(inp.num_rows, int(budget_s / 3 / per_row)))
    n -= n % max(1, min(n, 4))
    sample = rows[:max(n, 1)]
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        lg = oracle.paged_logits(inp, rows=sample)
        oracle.topk(lg.astype(np.float32), inp.ctx_lens[sample], inp.topk)
        times.append(time.perf_counter() - t0)
    per_call_us = statistics.median(times) * 1e6 * inp.num_rows / len(sample)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"value": round(per_call_us, 1), "unit": "µs/call", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": affinity,
            "sample": f"{len(sample)} of {inp.num_rows} rows (the first ones), scoring + top-k, median of 3, "
                      f"scaled by rows; float64 C loops, OpenMP over rows on {threads} threads"}


def _timed_region(step, steps, warmup, stream):
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    return t_start.elapsed_time(t_end)


def _settle(step, stream, ms=60.0):
    """Run `step` (untimed) for about `ms` milliseconds of GPU time, so that the
    clocks have settled before a timed region starts."""
    import torch
    step(0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    step(1)
    e1.record(stream)
    torch.cuda.synchronize()
    n = min(2000, max(1, math.ceil(ms / max(e0.elapsed_time(e1), 1e-3))))
    for i in range(n):
        step(i)
    torch.cuda.synchronize()


def measure(workload, steps, warmup):
    """Time `steps` calls of the workload (after `warmup`): the library's full
    call (qsa_paged_logits_topk: scoring then selection, fused where the shape
    allows), and the same work as two calls (qsa_paged_logits, qsa_topk) for
    comparison; then the full calls again with the scoring and the selection
    timed by their own dispatch events.  Returns the figures of one
    configuration (and the inputs)."""
    import torch

    import paged_mqa_logits_block_amd as qsa
    import qsa_inputs
    from qsa_inputs.device import to_device

    inp = qsa_inputs.make_config(workload)
    reads, writes = algorithmic_bytes(inp)
    per_call = reads + writes
    tk_reads, tk_writes = topk_bytes(inp)
    reps = max(1, min(16, math.ceil(600e6 / max(inp.kcache.nbytes + writes, 1))))
    devs = [to_device(inp) for _ in range(reps)]
    outs = [torch.empty((inp.num_rows, inp.width), dtype=torch.float32, device="cuda") for _ in range(reps)]
    idx = torch.empty((inp.num_rows, inp.topk), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    # calls validated once per replica; a step only crosses the C ABI
    full, two = [], []
    for d, o in zip(devs, outs):
        full.append(qsa.PreparedLogitsTopk(d.q, d.kcache, d.block_table, d.ctx_lens, d.row_to_req, o, idx,
                                           k=d.topk, width=d.width, block_size=d.block_size, w=d.w,
                                           kscale=d.kscale, layout=d.layout, stream=stream))
        two.append((qsa.PreparedLogits(d.q, d.kcache, d.block_table, d.ctx_lens, d.row_to_req, o,
                                       width=d.width, block_size=d.block_size, w=d.w, kscale=d.kscale,
                                       layout=d.layout, stream=stream),
                    qsa.PreparedTopk(o, d.ctx_lens, d.topk, idx, stream=stream)))

    def step_full(i):
        full[i % reps]()

    def step_two(i):
        lg, tk = two[i % reps]
        lg()
        tk()

    # both paths run untimed first, alternately, for about 60 ms: the GPU's
    # clocks settle over tens of milliseconds of work, and the first timed
    # region would otherwise start cold.  The two-call step takes the replica
    # half the set away, so that it does not read keys the full call has just
    # brought into the Infinity Cache (kernel traces count these dispatches)
    _settle(lambda i: (step_full(i), step_two(i + reps // 2)), stream)
    # timed region: exactly K steps, events only around the whole region
    total_ms = _timed_region(step_full, steps, warmup, stream)
    two_ms = _timed_region(step_two, steps, max(1, warmup // 2), stream)

    # kernel durations: the same K steps again, the scoring and the selection
    # timed by HIP events that their own dispatches record (on the stream the
    # kernels run on); these events add host and GPU time per launch, so they
    # stay out of the regions above
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e3 in evs:
        for e in e3:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        full[i % reps](evs[i])
    torch.cuda.synchronize()
    logit_us = statistics.mean(e[0].elapsed_time(e[1]) for e in evs) * 1e3
    topk_us = statistics.mean(e[1].elapsed_time(e[2]) for e in evs) * 1e3
    fused = full[0].workspace is not None and full[0].workspace.numel() > 0 and inp.num_heads <= 4 \
        and scoring_kernel(inp) == "paged_logits_kernel"

    sk = scoring_kernel(inp)
    s_gbs = per_call / (logit_us * 1e-6) / 1e9
    scoring = {"kernel": sk + (" (+ chunk candidates)" if fused else ""), "bound": "hbm",
               "us": round(logit_us, 2), "achieved": round(s_gbs, 1),
               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(s_gbs / HBM_PEAK_GBS, 4),
               "traffic": measured_traffic(workload, sk), "algorithmic_bytes": per_call,
               "algorithmic_read_bytes": reads, "algorithmic_write_bytes": writes}
    flops = scoring_flops(inp)
    tflops = flops / (logit_us * 1e-6) / 1e12
    peak_tf = MFMA_PEAK_TFLOPS[inp.dtype]
    scoring["mfma"] = {"achieved": round(tflops, 1), "peak": peak_tf, "unit": "TFLOP/s",
                       "frac": round(tflops / peak_tf, 4), "algorithmic_flops": flops,
                       "busy_frac_counters": measured_mfma_busy(workload, sk)}
    tplan = topk_plan(inp)
    t_gbs = (tk_reads + tk_writes) / (topk_us * 1e-6) / 1e9
    tkname = ("topk_cand_kernel" if fused else
              "topk_window_kernel + topk_resolve_kernel" if tplan == "split" else "topk_rows_kernel")
    topk = {"kernel": tkname, "bound": "hbm", "us": round(topk_us, 2), "achieved": round(t_gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(t_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(workload, "topk"),
            "algorithmic_bytes": tk_reads + tk_writes, "algorithmic_read_bytes": tk_reads,
            "algorithmic_write_bytes": tk_writes}
    res = {"workload": workload, "value": round(total_ms * 1e3 / steps, 2), "ms_per_step": total_ms / steps,
           "two_call_value": round(two_ms * 1e3 / steps, 2), "fused": fused,
           "logits_us": round(logit_us, 2), "topk_us": round(topk_us, 2), "scoring": scoring, "topk": topk,
           "replicas": reps, "steps": steps, "warmup": warmup}
    del full, two, devs, outs, idx
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, inp


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_chunk", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the summary runs of the five workloads")
    ap.add_argument("--config-steps", type=int, default=30, help="timed steps per summary run")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CALIB_FETCH_DIR",
                                                          "CALIB_WRITE_DIR"),
                    help="record a kernel's counter bytes from rocprofv3 --pmc output folders "
                         "(FETCH_SIZE, WRITE_SIZE, and both for a --calib-copy-mib run); no GPU needed")
    ap.add_argument("--kernel", default="scoring", choices=["scoring", "topk"],
                    help="which kernel --write-traffic records")
    ap.add_argument("--write-mfma", metavar="DIR",
                    help="record the scoring kernel's MFMA busy fraction from a rocprofv3 --pmc "
                         "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE output folder; no GPU needed")
    ap.add_argument("--calib-mib", type=int, default=1024, help="size of the calibration copy")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the scoring path has no multi-GPU variant in this library)", file=sys.stderr)
        sys.exit(2)

    if args.write_traffic or args.write_mfma:
        import qsa_inputs
        inp = qsa_inputs.make_config(args.workload)
        if args.write_traffic:
            k = "topk" if args.kernel == "topk" else scoring_kernel(inp)
            write_traffic(args.workload, k, args.write_traffic, args.calib_mib)
        if args.write_mfma:
            write_mfma(args.workload, scoring_kernel(inp), args.write_mfma)
        return

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

    import qsa_inputs

    head, inp = measure(args.workload, args.steps, args.warmup)
    kernels = [head["scoring"], head["topk"]]
    dom = max(kernels, key=lambda e: e["us"])
    roofline = {k: dom[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel",
                                    "algorithmic_bytes", "algorithmic_read_bytes", "algorithmic_write_bytes")}
    roofline["kernels"] = kernels
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic (seeded generators; shapes of the pages' workloads)",
        "config": {"workload": args.workload, "description": DESCRIPTIONS[args.workload],
                   "rows": inp.num_rows, "width": inp.width, "heads": inp.num_heads,
                   "block": inp.block_size, "topk": inp.topk, "input_replicas": head["replicas"]},
        "logits_us": head["logits_us"],
        "topk_us": head["topk_us"],
        "two_call_value": head["two_call_value"],
        "fused_selection": head["fused"],
        "roofline": roofline,
    }
    if not args.no_configs:
        summary = []
        for name in qsa_inputs.CONFIG_NAMES:
            r = head if name == args.workload else measure(name, args.config_steps, 5)[0]
            summary.append({"workload": name, "value": r["value"], "two_call_value": r["two_call_value"],
                            "fused_selection": r["fused"], "logits_us": r["logits_us"],
                            "topk_us": r["topk_us"], "scoring_kernel": r["scoring"]["kernel"],
                            "scoring_frac": r["scoring"]["frac"],
                            "scoring_mfma_frac": r["scoring"]["mfma"]["frac"],
                            "scoring_traffic": r["scoring"]["traffic"],
                            "topk_kernel": r["topk"]["kernel"], "topk_frac": r["topk"]["frac"],
                            "steps": r["steps"]})
            print(f"[config] {json.dumps(summary[-1])}", file=sys.stderr, flush=True)
        line["configs"] = summary
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
