"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case prints what it runs before the first launch, so a failing run names
its case.  Inputs come from qsa_inputs (seeded); expected values only from the
oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import qsa_inputs
from gpu_helpers import (TOPK_PATHS, qsa, assert_logits_match, assert_topk_banded, assert_topk_exact,
                         gpu_logits, gpu_topk)
from qsa_inputs.device import to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mqa_logits_block_amd as m
    say("library", m.version(), "device", torch.cuda.get_device_name(0))
    return m


def run_logits(inp, **kw):
    dev = to_device(inp)
    g = gpu_logits(inp, dev, **kw)
    torch.cuda.synchronize()
    return dev, g


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def _prefill_sample_rows(n=16384):
    """One whole 128-row tile of the prefill scoring kernel, every 16th row after
    it (other tiles, both halves of each consumer wave's rows), and the last."""
    return sorted(set(range(128)) | set(range(128, n, 16)) | {n - 1})


SAMPLED_ROWS = {"prefill_chunk": _prefill_sample_rows()}
SAMPLED_ROWS["prefill_chunk_fp16"] = SAMPLED_ROWS["prefill_chunk"]


@pytest.mark.parametrize("name", qsa_inputs.CONFIG_NAMES + qsa_inputs.FP16_CONFIG_NAMES +
                         qsa_inputs.KVB1_CONFIG_NAMES + qsa_inputs.SHUFFLED_CONFIG_NAMES +
                         qsa_inputs.D64_CONFIG_NAMES + qsa_inputs.RAGGED_CONFIG_NAMES)
def test_config_logits_and_topk(name):
    inp = qsa_inputs.make_config(name, poison=True)
    rows = SAMPLED_ROWS.get(name)
    say(name, "rows", inp.num_rows, "width", inp.width, "H", inp.num_heads, inp.dtype, inp.layout,
        "compared rows", inp.num_rows if rows is None else len(rows))
    dev, g = run_logits(inp)
    sel = list(range(inp.num_rows)) if rows is None else rows
    o = oracle.paged_logits(inp, rows=sel)
    gl = g[torch.tensor(sel, device="cuda")].cpu().numpy()
    tols = assert_logits_match(gl, o, inp, sel, label=name)

    # top-k on the GPU's own logits (all rows in one call, as the benchmark
    # runs it), end to end, against the oracle's selection
    gi = gpu_topk(g, dev.ctx_lens, inp.topk)[torch.tensor(sel, device="cuda")].cpu().numpy()
    o32 = o.astype(np.float32)
    oi = oracle.topk(o32, inp.ctx_lens[sel], inp.topk)
    assert_topk_banded(gi, oi, o, tols, label=name)

    # top-k on identical logits (the oracle's, uploaded; every compared row in
    # one call): exact, on both selection paths where the shape has two
    lt = torch.from_numpy(np.ascontiguousarray(o32)).cuda()
    ct = torch.from_numpy(inp.ctx_lens[sel].astype(np.int32)).cuda()
    for path, ws in TOPK_PATHS.items():
        gi2 = gpu_topk(lt, ct, inp.topk, workspace=ws).cpu().numpy()
        assert_topk_exact(gi2, oi, label=f"{name} {path}")
        # ascending column order, -1 padding after the selection
        for r in range(gi2.shape[0]):
            v = gi2[r][gi2[r] >= 0]
            assert np.all(np.diff(v) > 0)
            assert np.all(gi2[r][len(v):] == -1)


# ---------------------------------------------------------------------------
# logits edge cases
# ---------------------------------------------------------------------------

EDGE_CTX = [0, 1, 15, 16, 17, 63, 64, 65, 255, 256, 257, 1000]


@pytest.mark.parametrize("H", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("dtype,layout", [("bf16", "paged"), ("fp16", "paged"), ("fp8", "paged"),
                                          ("fp8", "copacked"), ("fp8", "copacked_shuffled")])
def test_heads_and_dtypes(H, dtype, layout):
    ctx = [EDGE_CTX[(i * 5 + H) % len(EDGE_CTX)] for i in range(6)]
    inp = qsa_inputs.build(name="edge", seed=100 + H, req_rows=[2, 1, 3], ctx_rows=ctx,
                           num_heads=H, block_size=16 if H < 16 else 64, dtype=dtype,
                           layout=layout, weights=(H % 2 == 0), poison=True)
    say("heads", H, dtype, layout, "ctx", ctx)
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label=f"H{H}")


@pytest.mark.parametrize("H", [16, 32, 64])
@pytest.mark.parametrize("layout", ["paged", "copacked"])
@pytest.mark.parametrize("req_rows", [(4, 4, 4, 4), (5, 3, 6, 2), (7, 8, 1, 3), (8, 8, 2)])
def test_fp8_many_heads_mtp_rows(H, layout, req_rows):
    """fp8, 16+ heads, 4+ rows per request (the MTP verify shape): ragged ctx
    within a request, requests of unequal row counts, a width that ends inside
    a key tile, poisoned table slots and key tails."""
    n = sum(req_rows)
    base = [1000, 997, 998, 999, 65, 64, 63, 0, 3000, 2999, 2998, 2997, 16, 17, 15, 1]
    ctx = [base[i % len(base)] for i in range(n)]
    inp = qsa_inputs.build(name="stack", seed=700 + H + n, req_rows=list(req_rows), ctx_rows=ctx,
                           num_heads=H, block_size=64, dtype="fp8", layout=layout,
                           weights=(H != 32), width=3004, poison=True)
    say("fp8 mtp rows", H, layout, req_rows)
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label=f"mtp H{H}")


@pytest.mark.parametrize("H", [32, 64])
@pytest.mark.parametrize("layout", ["paged", "copacked", "copacked_shuffled"])
@pytest.mark.parametrize("shuffle", [False, True])
def test_fp8_four_row_requests(H, layout, shuffle):
    """fp8, 32/64 heads, exactly 4 rows per request (the 4-row workgroup
    variant): ragged ctx inside a request, a width ending inside a key run,
    blocks of 64 and 128 columns, poisoned table slots and key tails; with
    shuffle the rows of a request are scattered over tiles (tiles whose rows
    belong to several requests)."""
    reqs = 6
    base = [3000, 2999, 2998, 2997, 65, 64, 63, 0, 1000, 997, 998, 999, 129, 128, 127, 1,
            1500, 1499, 1498, 1497, 2048, 2047, 2046, 2045]
    ctx = base[:4 * reqs]
    B = 64 if H == 64 else 128
    inp = qsa_inputs.build(name="mtp4", seed=800 + H + (7 if shuffle else 0), req_rows=[4] * reqs,
                           ctx_rows=ctx, num_heads=H, block_size=B, dtype="fp8", layout=layout,
                           weights=True, width=3004, poison=True, shuffle_rows=shuffle)
    say("fp8 4-row requests", H, layout, "shuffle", shuffle)
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label=f"mtp4 H{H}")


@pytest.mark.parametrize("reqs,B,layout,shuffle", [
    (40, 64, "copacked", False),    # ~180 rows grouped by request: tiles follow the requests
    (40, 128, "copacked_shuffled", False),
    (40, 3, "paged", False),        # the same with blocks of 3 columns (gather)
    (40, 64, "copacked", True),     # rows scattered: more tiles than the grid holds, plain tiles
    (57, 64, "paged", False),       # exactly 256 rows
    (70, 64, "copacked", False),    # past 256 rows: plain tiles walking the requests
])
def test_fp8_ragged_verify_rows(reqs, B, layout, shuffle):
    """fp8, 64 heads, 1..8 verify rows per request (ragged next_n): the 4-row
    variant with tiles cut from each request's first row, its fallback to plain
    tiles for rows not grouped by request, and plain tiles past 256 rows."""
    rng = np.random.default_rng(900 + reqs + B)
    if reqs == 57:
        counts = np.array([5] * 32 + [1] * 4 + [5] * 8 + [4] * 13)
        assert counts.sum() == 256
    else:
        counts = rng.integers(1, 9, size=reqs)
    n = int(counts.sum())
    # row j of a request with nn rows and kv_len keys sees kv_len - nn + j + 1
    ctx = []
    for nn in counts:
        kv_len = int(rng.integers(1, 3005))
        ctx += [max(kv_len - int(nn) + j + 1, 0) for j in range(int(nn))]
    inp = qsa_inputs.build(name="ragged", seed=950 + reqs + B, req_rows=[int(c) for c in counts],
                           ctx_rows=ctx, num_heads=64, block_size=B, dtype="fp8",
                           layout=layout, weights=True, width=3004, poison=True, shuffle_rows=shuffle)
    say("fp8 ragged rows", reqs, n, B, layout, "shuffle", shuffle)
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label=f"ragged R{n} B{B}")


@pytest.mark.parametrize("B", [1, 3, 100])
@pytest.mark.parametrize("H,layout", [(64, "copacked"), (32, "paged")])
@pytest.mark.parametrize("shuffle", [False, True])
def test_fp8_four_row_requests_gather(B, H, layout, shuffle):
    """The 4-row fp8 variant with blocks that do not hold whole 64-column runs
    (down to one key per block): table entries staged per column, each key
    fetched from its own block, validity per column."""
    reqs = 5
    ctx = [3000, 2999, 2998, 2997, 65, 64, 63, 0, 1000, 997, 998, 999, 129, 128, 127, 1,
           1500, 1499, 1498, 1497]
    inp = qsa_inputs.build(name="mtp4 gather", seed=860 + B + H + (3 if shuffle else 0), req_rows=[4] * reqs,
                           ctx_rows=ctx, num_heads=H, block_size=B, dtype="fp8", layout=layout,
                           weights=True, width=3004, poison=True, shuffle_rows=shuffle)
    say("fp8 4-row gather", B, H, layout, "shuffle", shuffle)
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label=f"mtp4 gather B{B} H{H}")


def test_fp8_four_row_requests_long():
    """The 4-row fp8 variant at a size where each workgroup walks several key
    runs (16 requests x 16,384 columns: 4 runs of 64 columns per workgroup,
    one full turn of the fetch ring), with an invalid table entry and an
    invalid request (NaN); the oracle checks sampled rows."""
    reqs, W = 16, 16384
    ctx = [W - (i % 4) * 37 for i in range(4 * reqs)]
    inp = qsa_inputs.build(name="mtp4 long", seed=880, req_rows=[4] * reqs, ctx_rows=ctx, kv_lens=[W] * reqs,
                           num_heads=64, block_size=64, dtype="fp8", layout="copacked", weights=True,
                           width=W)
    inp.block_table[1, 5] = inp.num_blocks + 2  # columns 320..383 of request 1
    inp.row_to_req = inp.row_to_req.copy()
    inp.row_to_req[10] = reqs + 3  # past the table
    say("fp8 4-row long, invalid entry / request")
    _, g = run_logits(inp)
    x = g.cpu().numpy()
    assert np.all(np.isnan(x[4:8, 320:384])) and np.all(np.isfinite(x[4:8, :320]))
    assert np.all(np.isnan(x[10, :ctx[10]])) and np.all(x[10, ctx[10]:] == -np.inf)
    rows = [0, 1, 2, 3, 8, 9, 11, 30, 63]
    o = oracle.paged_logits(inp, rows=rows)
    assert_logits_match(x[rows], o, inp, rows, label="mtp4 long")


@pytest.mark.parametrize("B", [16, 32, 64, 128, 1024])
def test_block_sizes_and_ragged_ctx(B):
    ctx = [1, B - 1, B, B + 1, 3 * B + 5, 2047, 2048, 2049]
    inp = qsa_inputs.build(name="blk", seed=200 + B, req_rows=[4, 4], ctx_rows=ctx, num_heads=4,
                           block_size=B, poison=True)
    say("block", B, "ctx", ctx)
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label=f"B{B}")


@pytest.mark.parametrize("B", [48, 80, 400])
@pytest.mark.parametrize("dtype,layout,H", [("bf16", "paged", 4), ("bf16", "paged", 16), ("fp16", "paged", 4),
                                            ("fp8", "paged", 16), ("fp8", "copacked", 64)])
def test_page_sizes_not_powers_of_two(B, dtype, layout, H):
    """Block sizes that are multiples of 16 but not powers of two (page size
    400 of the pages' callers): tiles and key groups straddle block edges at
    other offsets, and 64-column key runs do not fit a block evenly."""
    ctx = [1, B - 1, B, B + 1, 2 * B + 17, 5 * B, 3001, 4099]
    inp = qsa_inputs.build(name="blkodd", seed=400 + B + H, req_rows=[3, 1, 4], ctx_rows=ctx,
                           num_heads=H, block_size=B, dtype=dtype, layout=layout, weights=True, poison=True)
    say("odd block", B, dtype, layout, H, "ctx", ctx)
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label=f"B{B} {dtype} {layout} H{H}")


@pytest.mark.parametrize("B", [1, 3, 7, 17, 100])
@pytest.mark.parametrize("dtype,layout,H", [("bf16", "paged", 4), ("fp16", "paged", 2), ("bf16", "paged", 16),
                                            ("fp8", "paged", 16), ("fp8", "copacked", 64)])
def test_block_sizes_not_multiples_of_16(B, dtype, layout, H):
    """Block sizes down to one key per table entry (the per-token layout): a
    16-column tile straddles blocks, every lane gathers its own column.  The
    tables are seeded permutations, so neighbouring columns sit in unrelated
    blocks; contexts end inside and at the edges of blocks and tiles."""
    ctx = [1, 2, B, B + 1, 15, 16, 17, 33 * B + 5, 1000, 1999]
    inp = qsa_inputs.build(name="blkgather", seed=700 + B + H, req_rows=[4, 2, 4], ctx_rows=ctx,
                           num_heads=H, block_size=B, dtype=dtype, layout=layout, weights=True, poison=True)
    say("gather block", B, dtype, layout, H, "ctx", ctx)
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label=f"B{B} {dtype} {layout} H{H}")


def test_block_size_one_invalid_entry_gives_nan_in_its_column_only():
    """With one key per block a bad table entry spoils exactly its column."""
    inp = qsa_inputs.build(name="blk1 bad", seed=771, req_rows=[4], ctx_rows=[300] * 4, kv_lens=[300],
                           num_heads=4, block_size=1)
    inp.block_table[0, 37] = inp.num_blocks + 5
    say("block 1 invalid entry")
    _, g = run_logits(inp)
    x = g.cpu().numpy()
    assert np.all(np.isnan(x[:, 37]))
    keep = np.ones(inp.width, dtype=bool)
    keep[37] = False
    o = oracle.paged_logits(inp.__class__(**{**inp.__dict__, "block_table": np.where(
        inp.block_table >= inp.num_blocks, 0, inp.block_table).astype(np.int32)}))
    assert np.all(np.isfinite(x[:, :300][:, keep[:300]]))
    d = np.abs(x[:, :300][:, keep[:300]].astype(np.float64) - o[:, :300][:, keep[:300]])
    assert np.all(d <= 5e-5 + 5e-5 * np.abs(o[:, :300][:, keep[:300]]))


@pytest.mark.parametrize("dtype,layout", [("bf16", "paged"), ("fp16", "paged"), ("fp8", "paged"),
                                          ("fp8", "copacked"), ("fp8", "copacked_shuffled")])
@pytest.mark.parametrize("H,B,req_rows", [(4, 16, [4, 4, 4]), (16, 64, [4, 4, 4]), (64, 16, [4, 4, 4]),
                                          (2, 3, [3, 1, 5]), (64, 48, [1, 2, 2])])
def test_head_dim_64(dtype, layout, H, B, req_rows):
    """Head dim 64 (the per-tile kernel for every shape): zero K steps for
    bf16/fp16, zero lane groups in the fp8 MFMA; 4-row requests and many heads
    that take other kernels at D = 128; block sizes with the per-column gather."""
    R = sum(req_rows)
    ctx = [[1, 15, 16, 17, 64, 65, 1000, 1999, 2000, 7, 33, 500][i % 12] for i in range(R)]
    if layout == "copacked_shuffled" and B % 16:
        # the preshuffled layout is defined for blocks of a multiple of 16
        # columns: the call is refused before any launch
        m = qsa()
        inp = qsa_inputs.build(name="d64", seed=300 + H + B, req_rows=req_rows, ctx_rows=ctx, num_heads=H,
                               head_dim=64, block_size=B, dtype=dtype, layout="copacked", weights=True)
        dev = to_device(inp)
        say("head dim 64 refused", dtype, layout, "H", H, "B", B)
        with pytest.raises(m.QsaError) as e:
            m.paged_logits(dev.q, dev.kcache, dev.block_table, dev.ctx_lens, dev.row_to_req, width=dev.width,
                           block_size=B, w=dev.w, layout=m.KV_COPACKED_SHUFFLED)
        assert e.value.status == m.E_UNSUPPORTED
        return
    inp = qsa_inputs.build(name="d64", seed=300 + H + B, req_rows=req_rows, ctx_rows=ctx, num_heads=H,
                           head_dim=64, block_size=B, dtype=dtype, layout=layout, weights=True, poison=True)
    say("head dim 64", dtype, layout, "H", H, "B", B)
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label=f"D64 {dtype} {layout} H{H} B{B}")


def _prefill_ctx(n, W, seed):
    """Causal visible counts of a chunk of n rows ending at column W, with
    edge counts mixed in (0, 1, a step boundary and its neighbours, past the
    width)."""
    rng = np.random.default_rng(seed)
    ctx = (W - n + 1 + np.arange(n)).astype(np.int64)
    ctx = np.minimum(ctx, W)
    edges = [0, 1, 31, 32, 33, 63, 64, 65, W - 1, W, W + 100]
    at = rng.choice(n, size=len(edges), replace=False)
    ctx[at] = edges
    return ctx


@pytest.mark.parametrize("B", [32, 64, 128])
@pytest.mark.parametrize("weights", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_prefill_many_rows_one_request(B, weights, dtype):
    """bf16 or fp16, 4 heads, one request holding a few hundred rows (the
    prefill chunk shape, its own kernel): ragged row count and width, edge
    visible counts, poisoned table slots and key tails."""
    n, W = 333, 1000
    ctx = _prefill_ctx(n, W, seed=B)
    inp = qsa_inputs.build(name="prefill", seed=900 + B, req_rows=[n], ctx_rows=ctx, kv_lens=[W],
                           num_heads=4, block_size=B, width=W, weights=weights, dtype=dtype, poison=True)
    say("prefill rows", n, "width", W, "block", B, "weights", weights, dtype)
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label=f"prefill B{B}")


def test_prefill_long_column_range():
    """Prefill kernel with several 32-column steps per program (an odd count)
    and a width that ends inside a step."""
    n, W = 300, 20012
    ctx = _prefill_ctx(n, W, seed=7)
    inp = qsa_inputs.build(name="prefill", seed=951, req_rows=[n], ctx_rows=ctx, kv_lens=[W],
                           num_heads=4, block_size=64, width=W, weights=True, poison=True)
    say("prefill long rows", n, "width", W)
    _, g = run_logits(inp)
    rows = list(range(0, n, 7)) + [n - 1]
    x = g.cpu().numpy()[rows]
    assert_logits_match(x, oracle.paged_logits(inp, rows=rows), inp, rows, label="prefill long")


def test_prefill_invalid_table_entry_and_request_give_nan():
    n, W = 260, 512
    inp = qsa_inputs.build(name="prefill bad", seed=952, req_rows=[n], ctx_rows=[300] * n,
                           kv_lens=[W], num_heads=4, block_size=64, width=W)
    inp.block_table[0, 2] = inp.num_blocks + 3  # columns 128..191
    inp.row_to_req = inp.row_to_req.copy()
    inp.row_to_req[[5, 200]] = 1  # only request 0 exists
    say("prefill invalid table entry / request")
    _, g = run_logits(inp)
    x = g.cpu().numpy()
    ok = np.ones(n, bool)
    ok[[5, 200]] = False
    assert np.all(np.isnan(x[ok][:, 128:192])) and np.all(np.isfinite(x[ok][:, :128]))
    assert np.all(np.isfinite(x[ok][:, 192:300])) and np.all(x[:, 300:] == -np.inf)
    assert np.all(np.isnan(x[~ok][:, :300]))


def test_rows_spanning_requests_and_shuffled():
    # one row per request, and rows of one request scattered over tiles
    ctx = list(range(100, 100 + 37 * 13, 13))
    inp = qsa_inputs.build(name="span", seed=301, req_rows=[1] * 37, ctx_rows=ctx, num_heads=4,
                           block_size=16, weights=True, poison=True)
    say("spanning", len(ctx))
    _, g = run_logits(inp)
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label="span")
    inp2 = qsa_inputs.build(name="shuf", seed=302, req_rows=[3, 5, 2, 6], ctx_rows=[40 + 9 * i for i in range(16)],
                            num_heads=4, block_size=16, shuffle_rows=True, poison=True)
    say("shuffled rows")
    _, g2 = run_logits(inp2)
    assert_logits_match(g2.cpu().numpy(), oracle.paged_logits(inp2), inp2, label="shuf")


def test_ctx_clamping_and_width():
    # ctx beyond the table, beyond the width, and negative
    inp = qsa_inputs.build(name="clamp", seed=401, req_rows=[2, 2], ctx_rows=[5000, 70, -3, 64],
                           kv_lens=[64, 64], num_heads=4, block_size=16, max_blocks=4, width=50,
                           poison=True)
    say("clamp")
    dev = to_device(inp)
    # a ragged width needs a row stride padded to a multiple of 4 floats
    buf = torch.full((inp.num_rows, 52), float("nan"), dtype=torch.float32, device="cuda")
    gpu_logits(inp, dev, out=buf[:, :50])
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(np.isnan(b[:, 50:]))
    assert_logits_match(b[:, :50], oracle.paged_logits(inp), inp, label="clamp")
    m = pytest.importorskip("paged_mqa_logits_block_amd")
    with pytest.raises(m.QsaError) as e:
        gpu_logits(inp, dev, out=torch.empty((inp.num_rows, 50), dtype=torch.float32, device="cuda"))
    assert e.value.status == m.E_ALIGN  # unpadded stride 50
    # without `out` the binding pads the rows itself and returns the [R, 50] view
    g = gpu_logits(inp, dev)
    torch.cuda.synchronize()
    assert tuple(g.shape) == (inp.num_rows, 50) and g.stride(0) == 52
    assert_logits_match(g.cpu().numpy(), oracle.paged_logits(inp), inp, label="clamp padded")


def test_untouched_stride_tail_and_nan_canaries():
    inp = qsa_inputs.make_config("tiny", poison=True)
    dev = to_device(inp)
    stride = inp.width + 52
    buf = torch.full((inp.num_rows, stride), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[:, : inp.width]
    say("stride tail")
    gpu_logits(inp, dev, out=out)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(np.isnan(b[:, inp.width:]))
    assert_logits_match(b[:, : inp.width], oracle.paged_logits(inp), inp, label="stride")


@pytest.mark.parametrize("kind", ["prefill", "fp8_4row"])
def test_untouched_stride_tail_new_variants(kind):
    """Padded output rows for the prefill and 4-row fp8 variants: the columns
    between the width and the stride keep their NaN canaries (the prefill
    variant's range-checked stores drop lanes past the width), and the first
    canary column past the last row is untouched too."""
    if kind == "prefill":
        n, W = 300, 1000 + 4
        inp = qsa_inputs.build(name="prefill stride", seed=961, req_rows=[n], ctx_rows=_prefill_ctx(n, W, 3),
                               kv_lens=[W], num_heads=4, block_size=64, width=W, poison=True)
    else:
        inp = qsa_inputs.build(name="fp8 4-row stride", seed=962, req_rows=[4] * 5,
                               ctx_rows=[1000, 999, 998, 997] * 5, num_heads=64, block_size=64, dtype="fp8",
                               layout="copacked", weights=True, width=1004, poison=True)
    dev = to_device(inp)
    stride = inp.width + 44
    buf = torch.full((inp.num_rows + 1, stride), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[: inp.num_rows, : inp.width]
    say("stride tail", kind)
    gpu_logits(inp, dev, out=out)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(np.isnan(b[: inp.num_rows, inp.width:]))
    assert np.all(np.isnan(b[inp.num_rows]))
    rows = list(range(0, inp.num_rows, 7)) + [inp.num_rows - 1]
    assert_logits_match(b[rows, : inp.width], oracle.paged_logits(inp, rows=rows), inp, rows, label=kind)


def test_block_table_permutation_bitwise():
    inp = qsa_inputs.make_config("tiny")
    say("permutation")
    _, g1 = run_logits(inp)
    perm = np.random.default_rng(5).permutation(inp.num_blocks)
    inv = np.argsort(perm)
    inp.kcache = inp.kcache[inv]
    inp.block_table = perm[inp.block_table].astype(np.int32)
    _, g2 = run_logits(inp)
    assert torch.equal(g1, g2)


def test_repeat_launch_deterministic():
    inp = qsa_inputs.make_config("tiny")
    dev = to_device(inp)
    say("repeat")
    a = gpu_logits(inp, dev).clone()
    b = gpu_logits(inp, dev)
    ta = gpu_topk(a, dev.ctx_lens, 256).clone()
    tb = gpu_topk(b, dev.ctx_lens, 256)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ta, tb)


def test_invalid_table_entry_and_request_give_nan():
    inp = qsa_inputs.build(name="bad", seed=501, req_rows=[2, 2], ctx_rows=[40, 40, 40, 40],
                           num_heads=4, block_size=16)
    inp.block_table[0, 1] = inp.num_blocks + 7  # columns 16..31 of request 0
    inp.row_to_req = np.array([0, 0, 9, 1], dtype=np.int32)  # row 2 points past the table
    say("invalid table entry / request")
    _, g = run_logits(inp)
    x = g.cpu().numpy()
    assert np.all(np.isnan(x[0:2, 16:32])) and np.all(np.isfinite(x[0:2, :16]))
    assert np.all(np.isfinite(x[0:2, 32:40]))
    assert np.all(np.isnan(x[2, :40])) and np.all(x[2, 40:] == -np.inf)
    assert np.all(np.isfinite(x[3, :40]))


def test_empty_inputs():
    m = pytest.importorskip("paged_mqa_logits_block_amd")
    inp = qsa_inputs.make_config("tiny")
    dev = to_device(inp)
    say("empty")
    out = m.paged_logits(dev.q[:0], dev.kcache, dev.block_table, dev.ctx_lens[:0], dev.row_to_req[:0],
                         width=inp.width, block_size=16)
    assert out.shape == (0, inp.width)
    out2 = m.paged_logits(dev.q, dev.kcache, dev.block_table, dev.ctx_lens, dev.row_to_req,
                          width=0, block_size=16)
    assert out2.shape == (inp.num_rows, 0)
    lt = torch.zeros((0, 16), dtype=torch.float32, device="cuda")
    assert m.topk(lt, torch.zeros(0, dtype=torch.int32, device="cuda"), 8).shape == (0, 8)


# ---------------------------------------------------------------------------
# top-k edge cases (identical logits on both sides: exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", sorted(TOPK_PATHS))
@pytest.mark.parametrize("kind", ["normal", "ints", "const", "zeros", "relu", "offset", "tiny"])
@pytest.mark.parametrize("k", [1, 7, 256, 2048])
def test_topk_distributions(kind, k, path):
    W = 9000
    ctx = [0, 1, k - 1 if k > 1 else 0, k, k + 1, 3000, 8999, 9000, 12000, 4097]
    x = qsa_inputs.make_logits(len(ctx), W, ctx, seed=k * 7 + len(kind), kind=kind, tail="nan")
    say("topk", kind, k, path)
    xt = torch.from_numpy(x).cuda()
    ct = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    gi = gpu_topk(xt, ct, k, workspace=TOPK_PATHS[path]).cpu().numpy()
    ctx_np = np.minimum(np.maximum(np.array(ctx), 0), W)
    xo = x.copy()
    for r, c in enumerate(ctx_np):
        xo[r, c:] = -np.inf  # the oracle refuses NaN; the tail is never read
    oi = oracle.topk(xo, ctx_np, k)
    assert_topk_exact(gi, oi, label=f"{kind}/k{k}")


@pytest.mark.parametrize("path", sorted(TOPK_PATHS))
@pytest.mark.parametrize("W", [69632, 65600, 32768, 4096, 4099])
def test_topk_widths_and_large_tie_buckets(W, path):
    # const rows put everything in one bucket (larger than the LDS list);
    # ints rows make large tie groups inside the list
    rows = []
    for kind in ("const", "ints", "normal"):
        rows.append(qsa_inputs.make_logits(2, W, [W, W - 3], seed=W % 97, kind=kind))
    x = np.concatenate(rows)
    ctx = np.array([W, W - 3] * 3)
    say("topk width", W, path)
    stride = (W + 3) // 4 * 4  # rows padded to a multiple of 4 floats
    xt = torch.full((x.shape[0], stride), float("nan"), dtype=torch.float32, device="cuda")
    xt[:, :W] = torch.from_numpy(x).cuda()
    gi = gpu_topk(xt[:, :W], torch.from_numpy(ctx.astype(np.int32)).cuda(), 2048, width=W,
                  workspace=TOPK_PATHS[path]).cpu().numpy()
    oi = oracle.topk(x, ctx, 2048)
    assert_topk_exact(gi, oi, label=f"W{W}")


def _sampled_columns(n):
    """Columns the window selection samples from a row of n >= 2048 columns:
    128 runs of 16, centred at (2r+1) n / 256, clamped and aligned to 4."""
    cols = []
    for r in range(128):
        c = ((2 * r + 1) * n) // 256
        st = min(max(c - 8, 0), n - 16) & ~3
        cols.extend(range(st, st + 16))
    return np.unique(np.array(cols))


@pytest.mark.parametrize("rows,W,k", [(36, 29408, 2048), (128, 8192, 2048), (64, 65600, 2048),
                                      (5, 69632, 1), (17, 12000, 900), (2, 5000, 2047),
                                      (300, 9000, 2048), (260, 40000, 64)])
def test_topk_rows_shared_or_not(rows, W, k):
    """Few rows (split selection: each row shared by several workgroups) and
    many rows (one workgroup per row), ragged ctx, mixed distributions: both
    paths equal the oracle."""
    rng = np.random.default_rng(rows * 1000 + k)
    ctx = rng.integers(0, W + 1, size=rows)
    ctx[: min(rows, 3)] = [W, k + 1, max(k - 1, 0)][: min(rows, 3)]
    kinds = ["normal", "relu", "ints", "normal"]
    x = np.concatenate([qsa_inputs.make_logits(1, W, [int(ctx[r])], seed=r + 31, kind=kinds[r % 4])
                        for r in range(rows)])
    say("topk rows", rows, W, k)
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(ctx.astype(np.int32)).cuda()
    oi = oracle.topk(x, ctx, k)
    g = gpu_topk(xt, ct, k).cpu().numpy()
    assert_topk_exact(g, oi, label=f"rows {rows}")
    g1 = gpu_topk(xt, ct, k, workspace=None).cpu().numpy()
    assert_topk_exact(g1, oi, label=f"rows {rows} one workgroup per row")


@pytest.mark.parametrize("rows", [300, 600])
def test_topk_many_rows_infinities_and_fallbacks(rows):
    """Many rows per workgroup (rows > 256): finite rows take the register
    path; rows with +inf / -inf inside the visible range, one-value rows and
    rows of small integers (tie groups larger than the LDS list) are set aside
    and selected after the others; every row equals the oracle."""
    W, k = 9000, 2048
    rng = np.random.default_rng(rows)
    ctx = rng.integers(k - 50, W + 1, size=rows)
    ctx[::7] = W - 1  # a partial last float4 group
    kinds = ["normal", "relu", "ints", "const", "normal", "zeros"]
    x = np.concatenate([qsa_inputs.make_logits(1, W, [int(ctx[r])], seed=r, kind=kinds[r % 6])
                        for r in range(rows)])
    for r in range(0, rows, 11):
        n = int(ctx[r])
        cols = rng.integers(0, n, size=5)
        x[r, cols[:3]] = np.inf
        x[r, cols[3:]] = -np.inf
    say("topk many rows inf", rows)
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(ctx.astype(np.int32)).cuda()
    g = gpu_topk(xt, ct, k, workspace=None).cpu().numpy()
    assert_topk_exact(g, oracle.topk(x, ctx, k), label=f"many rows inf {rows}")


def test_topk_rows_map_from_previous_row():
    """One workgroup per row, rows r, r + 256, r + 512 in one workgroup: each row's
    histogram is first taken on the previous row's bucket map.  Rows shifted far
    above the previous row's range (every value in the top bucket), far below it
    (every value in the bottom bucket), much narrower inside it, and with an
    infinity after a finite row: the crossing stays exact, or the row
    falls back to its own map or the set-aside path; every row equals the oracle."""
    W, k, R = 9000, 2048, 1280
    rng = np.random.default_rng(4242)
    ctx = rng.integers(k + 1, W + 1, size=R)
    base = qsa_inputs.make_logits(R, W, ctx, seed=4243, kind="normal")
    x = base.copy()
    blk = np.arange(R) // 256
    vis = np.arange(W)[None, :] < ctx[:, None]
    x[blk == 1] = np.where(vis[blk == 1], x[blk == 1] + np.float32(1000.0), x[blk == 1])  # above
    x[blk == 2] = np.where(vis[blk == 2], x[blk == 2] - np.float32(5000.0), x[blk == 2])  # below
    x[blk == 3] = np.where(vis[blk == 3], x[blk == 3] * np.float32(1e-4), x[blk == 3])    # narrow
    for r in np.nonzero(blk == 4)[0][::5]:
        x[r, int(rng.integers(0, ctx[r]))] = np.float32(-np.inf) if r % 2 else np.float32(np.inf)
    x = x.astype(np.float32)
    say("topk map from previous row")
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(ctx.astype(np.int32)).cuda()
    g = gpu_topk(xt, ct, k, workspace=None).cpu().numpy()
    assert_topk_exact(g, oracle.topk(x, ctx, k), label="map from previous row")


def test_topk_rows_at_the_register_width():
    """One workgroup per row at the widest rows the register path holds (32,768
    columns: every float4 group of every thread live, the kept set's 128
    slices all full) and just past it (set aside), with rows just above k and
    a ragged last group, several rows per workgroup: every row equals the
    oracle."""
    W, k, R = 32768 + 16, 2048, 300
    rng = np.random.default_rng(3232)
    choices = np.array([32768, 32767, 32766, 32765, 32769, 32784, k + 1, k + 3, 4097, 30001])
    ctx = choices[rng.integers(0, len(choices), size=R)]
    kinds = ["normal", "relu", "normal", "offset"]
    x = np.concatenate([qsa_inputs.make_logits(1, W, [int(ctx[r])], seed=7000 + r, kind=kinds[r % 4])
                        for r in range(R)])
    say("topk rows at the register width")
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(ctx.astype(np.int32)).cuda()
    g = gpu_topk(xt, ct, k, workspace=None).cpu().numpy()
    assert_topk_exact(g, oracle.topk(x, ctx, k), label="register width")


def _tied_at_kth(x, n, k, rng, below, above, zero=False):
    """Row x (visible [0, n)): copies of its k-th largest value planted at
    `below` random columns from under it and `above` from over it, so that the
    column order has to cut a tie at the k-th value (the lowest columns of the
    tie group are kept).  zero: the row is first shifted so that the k-th value
    is 0.0, and the copies alternate between +0.0 and -0.0."""
    v = x[:n]
    order = np.argsort(-v, kind="stable")
    if zero:
        v -= v[order[k - 1]]
    t = v[order[k - 1]]
    cols = np.concatenate([rng.choice(order[k:], size=below, replace=False),
                           rng.choice(order[:k - 1], size=above, replace=False)])
    v[cols] = t
    if zero:
        v[cols[::2]] = np.float32(-0.0)
    return x


@pytest.mark.parametrize("rows,W", [(47, 32768), (48, 32768), (48, 32772), (128, 32768), (128, 32772)])
def test_topk_planner_row_rule_edges(rows, W):
    """Either side of the planner's rule (47 rows split, 48 rows of at most
    32,768 columns one workgroup per row, wider rows split again), with the
    automatic workspace, ragged counts, some rows at the full width and a tie
    at the k-th value past the cut in every third row: the workspace query says
    which path runs, and every row equals the oracle."""
    m = qsa()
    k = 2048
    rng = np.random.default_rng(rows * 100003 + W)
    ctx = rng.integers(k + 1, W + 1, size=rows)
    ctx[:3] = [W, W - 1, k + 1]
    x = (rng.standard_normal((rows, W)).astype(np.float32) * np.float32(10.0))
    for r in range(rows):
        x[r, int(ctx[r]):] = -np.inf
        if r % 3 == 0:
            _tied_at_kth(x[r], int(ctx[r]), k, rng, int(rng.integers(1, 50)), int(rng.integers(0, 5)))
    split = m.topk_workspace_bytes(rows, W, k) > 0
    assert split == (rows < 48 or W > 32768)
    say("topk planner edge", rows, W, "split" if split else "rows")
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(ctx.astype(np.int32)).cuda()
    g = gpu_topk(xt, ct, k).cpu().numpy()
    assert_topk_exact(g, oracle.topk(x, ctx, k), label=f"planner edge {rows}x{W}")


def test_topk_rows_tie_at_kth_cut_by_column():
    """Rows whose k-th value is repeated past the cut, on the register path (one
    workgroup per row, 2-3 rows per workgroup, each row's histogram on the
    previous row's map): 1..300 copies of it planted under it and 0..20 over it,
    some at columns before the k-th one's (more than 64 members in the crossing
    bucket take the radix select, fewer the one-wave ranking); ties of +0.0 and
    -0.0 at a k-th value of 0; each row equals the oracle (equal values kept in
    column order)."""
    W, k, R = 28672, 2048, 600
    rng = np.random.default_rng(4242)
    ctx = rng.integers(k + 64, W + 1, size=R)
    x = (rng.standard_normal((R, W)).astype(np.float32) * np.float32(10.0))
    for r in range(R):
        n = int(ctx[r])
        x[r, n:] = -np.inf
        below = int(rng.choice([1, 2, 3, 8, 20, 40, 100, 300]))
        above = int(rng.choice([0, 0, 1, 5, 20]))
        _tied_at_kth(x[r], n, k, rng, below, above, zero=(r % 10 == 9))
    say("topk rows tie at k-th cut by column")
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(ctx.astype(np.int32)).cuda()
    g = gpu_topk(xt, ct, k, workspace=None).cpu().numpy()
    assert_topk_exact(g, oracle.topk(x, ctx, k), label="tie at k-th")


def test_topk_sample_miss_falls_back():
    """Rows whose sampled columns are far below (or above) the rest: the
    sample's window misses the k-th value and the row takes the histogram
    selection; the result is unchanged."""
    W, k, rows = 20000, 2048, 8
    rng = np.random.default_rng(77)
    x = rng.standard_normal((rows, W)).astype(np.float32)
    ctx = np.array([W, W, 15000, 9000, 4500, 2100, W, 12345])
    for r in range(rows):
        n = int(min(ctx[r], W))
        if n >= 2048:
            sc = _sampled_columns(n)
            x[r, sc] = -1000.0 + rng.standard_normal(len(sc)).astype(np.float32)
        if r == 6:  # and one row where the sample sits far above the rest
            x[r, _sampled_columns(n)] = 1000.0
    say("topk sample miss")
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(ctx.astype(np.int32)).cuda()
    gs = gpu_topk(xt, ct, k).cpu().numpy()
    oi = oracle.topk(x, ctx, k)
    assert_topk_exact(gs, oi, label="sample miss")


def test_topk_workspace_reused_across_calls():
    """One workspace through several calls (different data and ctx, poisoned
    beforehand): each result equals the oracle; no state survives a call."""
    m = qsa()
    W, k, rows = 30000, 2048, 36
    nbytes = m.topk_workspace_bytes(rows, W, k)
    assert nbytes > 0
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    say("topk workspace reuse")
    for seed in (1, 2, 3):
        rng = np.random.default_rng(seed)
        ctx = rng.integers(k - 10, W + 1, size=rows).astype(np.int32)
        x = qsa_inputs.make_logits(rows, W, ctx, seed=seed, kind="normal")
        g = m.topk(torch.from_numpy(x).cuda(), torch.from_numpy(ctx).cuda(), k, workspace=ws).cpu().numpy()
        assert_topk_exact(g, oracle.topk(x, ctx, k), label=f"reuse {seed}")


def test_topk_padded_row_stride():
    W, stride = 5000, 5012
    x = qsa_inputs.make_logits(3, stride, [5000, 4000, 2500], seed=9, kind="normal", tail="nan")
    say("topk stride")
    xt = torch.from_numpy(x).cuda()[:, :W]
    ct = torch.tensor([5000, 4000, 2500], dtype=torch.int32, device="cuda")
    gi = gpu_topk(xt, ct, 2048, width=W).cpu().numpy()
    xo = x[:, :W].copy()
    xo[1, 4000:] = -np.inf
    xo[2, 2500:] = -np.inf
    oi = oracle.topk(xo, [5000, 4000, 2500], 2048)
    assert_topk_exact(gi, oi, label="stride")


def test_prepared_and_timed_calls_match():
    m = pytest.importorskip("paged_mqa_logits_block_amd")
    inp = qsa_inputs.make_config("tiny")
    dev = to_device(inp)
    say("prepared / timed calls")
    ref = gpu_logits(inp, dev).clone()
    ref_idx = gpu_topk(ref, dev.ctx_lens, inp.topk).clone()
    out = torch.full_like(ref, float("nan"))
    idx = torch.full_like(ref_idx, -7)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    pl = m.PreparedLogits(dev.q, dev.kcache, dev.block_table, dev.ctx_lens, dev.row_to_req, out,
                          width=inp.width, block_size=inp.block_size)
    pt = m.PreparedTopk(out, dev.ctx_lens, inp.topk, idx)
    pl((ev[0], ev[1]))
    pt((ev[2], ev[3]))
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(idx, ref_idx)
    assert ev[0].elapsed_time(ev[1]) > 0 and ev[2].elapsed_time(ev[3]) > 0
    pl()
    pt()
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(idx, ref_idx)


@pytest.mark.parametrize("name", ["tiny", "decode_verify", "fp8_paged"])
def test_graph_capture_replay(name):
    """Both calls captured into one HIP graph (scoring, then top-k with its
    workspace): every replay equals the eager result bit for bit, with eager
    calls on other inputs, into other outputs, between the replays."""
    m = qsa()
    inp = qsa_inputs.make_config(name)
    other = qsa_inputs.make_config(name, seed=77)
    dev, dev2 = to_device(inp), to_device(other)
    say("graph replay", name)
    s = torch.cuda.Stream()
    out = torch.empty((inp.num_rows, inp.width), dtype=torch.float32, device="cuda")
    idx = torch.empty((inp.num_rows, inp.topk), dtype=torch.int32, device="cuda")
    out2 = torch.empty((other.num_rows, other.width), dtype=torch.float32, device="cuda")
    idx2 = torch.empty((other.num_rows, other.topk), dtype=torch.int32, device="cuda")

    def calls(d, o, i):
        return (m.PreparedLogits(d.q, d.kcache, d.block_table, d.ctx_lens, d.row_to_req, o, width=d.width,
                                 block_size=d.block_size, w=d.w, kscale=d.kscale, layout=d.layout, stream=s),
                m.PreparedTopk(o, d.ctx_lens, d.topk, i, stream=s))

    lg, tk = calls(dev, out, idx)
    lg2, tk2 = calls(dev2, out2, idx2)
    torch.cuda.synchronize()
    lg()
    tk()
    torch.cuda.synchronize()
    ref, ref_idx = out.clone(), idx.clone()
    o_idx = oracle.topk(ref.cpu().numpy(), inp.ctx_lens, inp.topk)
    assert_topk_exact(idx.cpu().numpy(), o_idx, label=f"{name} eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lg()
        tk()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{name} replay {r}: logits differ"
        assert torch.equal(idx, ref_idx), f"{name} replay {r}: indices differ"
        lg2()  # eager work on other inputs between the replays
        tk2()
        torch.cuda.synchronize()


@pytest.mark.parametrize("rows", [3, 200])
def test_topk_range_too_narrow_for_buckets(rows):
    """Rows whose values all lie within 4,096 ulp of 1e-36 (a range below 1e-39):
    2,048 buckets over that range would need a scale beyond float32, so the
    whole row shares one bucket and the members are ranked exactly.  Visible
    counts just above k (at most 2,048: the register path ranks them from its
    member list) and far above it (the list overflows: the staged path)."""
    W, k = 6000, 300
    ctx = np.array([k + 1, 1000, 2048, 5999, W, 2049][: max(rows, 3)] * (rows // 3 + 1))[:rows]
    x = qsa_inputs.make_logits(rows, W, ctx, seed=rows, kind="tiny")
    say("topk tiny range", rows)
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(ctx.astype(np.int32)).cuda()
    oi = oracle.topk(x, ctx, k)
    for path, ws in TOPK_PATHS.items():
        gi = gpu_topk(xt, ct, k, workspace=ws).cpu().numpy()
        assert_topk_exact(gi, oi, label=f"tiny range {path}")


def test_topk_side_stream_auto_workspace():
    """topk(..., stream=s) with an automatic workspace: the workspace stays
    reserved for s until the selection has run there, so memory allocated and
    written on the current stream right after the call does not overlap it."""
    m = qsa()
    if not hasattr(torch.cuda, "_sleep"):
        pytest.skip("torch.cuda._sleep is not available")
    W, k, rows = 30000, 2048, 36
    rng = np.random.default_rng(41)
    ctx = rng.integers(k + 1, W + 1, size=rows).astype(np.int32)
    x = qsa_inputs.make_logits(rows, W, ctx, seed=41, kind="normal")
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(ctx).cuda()
    nbytes = m.topk_workspace_bytes(rows, W, k)
    assert nbytes > 0
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    say("topk side stream workspace")
    with torch.cuda.stream(s):
        torch.cuda._sleep(2_000_000)  # holds s for about a millisecond
    out = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    m.topk(xt, ct, k, out=out, stream=s)
    # current stream: allocate the workspace's size and fill it at once
    filler = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    filler.fill_(0x5A)
    torch.cuda.synchronize()
    assert bool(torch.all(filler == 0x5A)), "the selection wrote into memory handed out after the call"
    assert_topk_exact(out.cpu().numpy(), oracle.topk(x, ctx, k), label="side stream")


@pytest.mark.parametrize("name", ["tiny", "decode_verify", "fp8_paged"])
def test_graph_replay_new_inputs_in_place(name):
    """vLLM PR #62589, Validation: capture once, then replay with new queries
    and visible lengths written into the captured buffers.  Each replay equals
    the oracle on the new inputs (logits to the gate, top-k exact on the replay's
    own logits) and an eager call on the same buffers bit for bit."""
    import dataclasses

    m = qsa()
    inp = qsa_inputs.make_config(name)
    dev = to_device(inp)
    R, W, k = inp.num_rows, inp.width, inp.topk
    s = torch.cuda.Stream()
    out = torch.empty((R, W), dtype=torch.float32, device="cuda")
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    lg = m.PreparedLogits(dev.q, dev.kcache, dev.block_table, dev.ctx_lens, dev.row_to_req, out, width=W,
                          block_size=dev.block_size, w=dev.w, kscale=dev.kscale, layout=dev.layout, stream=s)
    tk = m.PreparedTopk(out, dev.ctx_lens, k, idx, stream=s)
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    say("graph replay, new inputs in place", name)
    with torch.cuda.stream(s):
        lg()
        tk()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lg()
        tk()
    torch.cuda.synchronize()
    for trial in range(3):
        rng = np.random.default_rng(5000 + trial)
        qf = rng.standard_normal(inp.q.shape).astype(np.float32)
        new_q = (qsa_inputs.f32_to_e4m3fn_codes(qf) if inp.dtype == "fp8"
                 else qsa_inputs.f32_to_bf16_bits(qf))
        # each row sees at most its request's keys
        cap = np.minimum(np.asarray(inp.kv_lens)[inp.row_to_req], W).astype(np.int64)
        new_ctx = (rng.random(R) * (cap + 1)).astype(np.int32)
        new_ctx[0], new_ctx[-1] = cap[0], max(0, min(int(cap[-1]), k - 1))
        inp2 = dataclasses.replace(inp, q=new_q, ctx_lens=new_ctx)
        dev2 = to_device(inp2)
        dev.q.copy_(dev2.q)
        dev.ctx_lens.copy_(dev2.ctx_lens)
        out.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        x = out.cpu().numpy()
        gi = idx.cpu().numpy()
        o = oracle.paged_logits(inp2)
        assert_logits_match(x, o, inp2, label=f"{name} replay {trial}")
        assert_topk_exact(gi, oracle.topk(x, new_ctx, k), label=f"{name} replay {trial}")
        ref, ref_idx = out.clone(), idx.clone()
        out.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            lg()
            tk()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(idx, ref_idx), f"{name} replay {trial}: eager differs"


# ---------------------------------------------------------------------------
# row starts and expand
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", sorted(TOPK_PATHS))
@pytest.mark.parametrize("rows,W", [(36, 30000), (9, 9000), (300, 9000)])
@pytest.mark.parametrize("aligned", [True, False])
def test_topk_row_starts(rows, W, aligned, path):
    """Per-row starts (sglang PR #48649 test body): each row's candidates are
    the columns [s, s + n) of a shared buffer, reported as offsets from s;
    starts that are multiples of 4 and starts that are not, starts past the
    width, ranges cut by the width, rows that fit in k; NaN outside every
    range.  Identical logits: exact against the oracle."""
    k = 2048
    rng = np.random.default_rng(rows * 31 + W + (0 if aligned else 7))
    n = rng.integers(0, W // 2, size=rows)
    n[: min(rows, 4)] = [W // 2, k + 1, k, 5][: min(rows, 4)]
    s = rng.integers(0, W // 2, size=rows)
    if aligned:
        s &= ~3
    else:
        s[::2] |= 1
    if rows > 6:
        s[5], n[5] = W + 10, 100        # start past the width: empty
        s[6], n[6] = W - 1000, 5000     # range cut by the width: 1000 columns
    kinds = ["normal", "ints", "const", "relu"]
    base = np.concatenate([qsa_inputs.make_logits(1, W, [W], seed=r + 77, kind=kinds[r % 4]) for r in range(rows)])
    x = np.full((rows, W), np.nan, dtype=np.float32)
    for r in range(rows):
        st = int(min(max(s[r], 0), W))
        m = int(min(max(n[r], 0), W - st))
        x[r, st:st + m] = base[r, st:st + m]
    say("topk row starts", rows, W, "aligned" if aligned else "unaligned", path)
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(n.astype(np.int32)).cuda()
    stt = torch.from_numpy(s.astype(np.int32)).cuda()
    oi = oracle.topk(x, n, k, row_starts=s)
    gi = gpu_topk(xt, ct, k, workspace=TOPK_PATHS[path], row_starts=stt).cpu().numpy()
    assert_topk_exact(gi, oi, label=f"row starts {rows}x{W}")
    for r in range(rows):  # ascending offsets, -1 padding after them
        v = gi[r][gi[r] >= 0]
        assert np.all(np.diff(v) > 0) and np.all(gi[r][len(v):] == -1)


def test_topk_row_starts_zero_equals_none():
    """All-zero starts select exactly what no starts select, on every path."""
    W, rows = 12000, 20
    rng = np.random.default_rng(5)
    ctx = rng.integers(0, W + 1, size=rows).astype(np.int32)
    x = qsa_inputs.make_logits(rows, W, ctx, seed=5, kind="normal")
    xt = torch.from_numpy(x).cuda()
    ct = torch.from_numpy(ctx).cuda()
    zero = torch.zeros(rows, dtype=torch.int32, device="cuda")
    say("topk zero starts")
    for path, ws in TOPK_PATHS.items():
        a = gpu_topk(xt, ct, 2048, workspace=ws)
        b = gpu_topk(xt, ct, 2048, workspace=ws, row_starts=zero)
        torch.cuda.synchronize()
        assert torch.equal(a, b), path


@pytest.mark.parametrize("ratio", [1, 4, 7])
@pytest.mark.parametrize("bounded", [False, True])
def test_expand(ratio, bounded):
    """qsa_expand against the oracle, bit for bit: selections of various fill
    (full, partial, empty rows), with and without a token bound."""
    m = qsa()
    rng = np.random.default_rng(ratio * 10 + bounded)
    R, k = 37, 2048
    idx = np.full((R, k), -1, np.int32)
    for r in range(R):
        cnt = [k, 0, 1, 100][r % 4] if r < 8 else int(rng.integers(0, k + 1))
        idx[r, :cnt] = np.sort(rng.choice(70000, size=cnt, replace=False))
    tl = rng.integers(0, 70000 * ratio, size=R).astype(np.int32) if bounded else None
    say("expand", ratio, "bounded" if bounded else "no bound")
    it = torch.from_numpy(idx).cuda()
    tt = None if tl is None else torch.from_numpy(tl).cuda()
    got = m.expand(it, ratio, token_lens=tt).cpu().numpy()
    assert np.array_equal(got, oracle.expand(idx, ratio, token_lens=tl))


def test_select_score_topk_expand_decode_verify():
    """The full selection on the decode-verify workload: scoring, top-k and
    expand (ratio 4, each row's token count 4 x its visible columns minus 3) as
    three calls; the top-k is exact on the GPU's own logits, the expand bit-exact
    on the GPU's own selection."""
    m = qsa()
    inp = qsa_inputs.make_config("decode_verify")
    say("select decode_verify")
    dev, g = run_logits(inp)
    idx = gpu_topk(g, dev.ctx_lens, inp.topk)
    tl = (4 * inp.ctx_lens.astype(np.int64) - 3).astype(np.int32)
    toks = m.expand(idx, 4, token_lens=torch.from_numpy(tl).cuda()).cpu().numpy()
    gi = idx.cpu().numpy()
    assert_topk_exact(gi, oracle.topk(g.cpu().numpy(), inp.ctx_lens, inp.topk), label="select")
    assert np.array_equal(toks, oracle.expand(gi, 4, token_lens=tl))


# ---------------------------------------------------------------------------
# fused scoring + selection (qsa_paged_logits_topk)
# ---------------------------------------------------------------------------

def _fused_vs_two_calls(inp, label, workspace="auto"):
    """The fused call's logits and indices against qsa_paged_logits followed by
    qsa_topk (workspace "auto"), bit for bit, and its indices against the oracle's
    selection on those same logits, exactly."""
    m = qsa()
    dev = to_device(inp)
    R, W, k = inp.num_rows, inp.width, inp.topk
    g1 = gpu_logits(inp, dev)
    i1 = gpu_topk(g1, dev.ctx_lens, k)
    g2, i2 = m.paged_logits_topk(dev.q, dev.kcache, dev.block_table, dev.ctx_lens, dev.row_to_req, k=k,
                                 width=W, block_size=dev.block_size, w=dev.w, kscale=dev.kscale,
                                 layout=dev.layout, workspace=workspace)
    torch.cuda.synchronize()
    assert torch.equal(g1, g2), f"{label}: logits differ"
    assert torch.equal(i1, i2), f"{label}: indices differ from the two calls"
    x = g2.cpu().numpy()
    assert_topk_exact(i2.cpu().numpy(), oracle.topk(x, inp.ctx_lens, k), label=label)
    return g2, i2


@pytest.mark.parametrize("name", ["tiny", "decode_verify", "decode_verify_fp16", "decode_verify_d64",
                                  "single_row_mixed", "fp8_paged", "fp8_paged_ragged", "fp8_paged_kvb1",
                                  "fp8_paged_shuffled"])
def test_fused_selection_workloads(name):
    inp = qsa_inputs.make_config(name)
    say("fused", name)
    g, i = _fused_vs_two_calls(inp, f"fused {name}")
    # and against the oracle's logits, end to end
    o = oracle.paged_logits(inp)
    tols = assert_logits_match(g.cpu().numpy(), o, inp, label=f"fused {name}")
    oi = oracle.topk(o.astype(np.float32), inp.ctx_lens, inp.topk)
    assert_topk_banded(i.cpu().numpy(), oi, o, tols, label=f"fused {name}")


@pytest.mark.parametrize("H,layout,B", [(64, "copacked", 64), (32, "paged", 128), (64, "copacked_shuffled", 64),
                                        (64, "copacked", 3), (32, "paged", 1)])
@pytest.mark.parametrize("req_rows", [(4, 4, 4, 4), (7, 8, 1, 3, 2)])
def test_fused_selection_four_row_fp8(H, layout, B, req_rows):
    """The full call (qsa_paged_logits_topk) on the 4-row fp8 scorer's shapes,
    where scoring and selection run unfused inside the one call: 4-row and
    ragged requests (tiles that follow the requests), block-flat, paged,
    preshuffled and gathered keys, a row that fits in k; against the two calls
    bit for bit."""
    n = sum(req_rows)
    rng = np.random.default_rng(1200 + H + B + n)
    ctx = []
    for nn in req_rows:
        kv_len = int(rng.choice([1500, 2100, 5000, 9000, 12288]))
        ctx += [kv_len - nn + j + 1 for j in range(nn)]
    ctx[0] = 700  # a row that fits in k
    inp = qsa_inputs.build(name="fused mtp", seed=1300 + H + B + n, req_rows=list(req_rows), ctx_rows=ctx,
                           num_heads=H, block_size=B, dtype="fp8", layout=layout, weights=True,
                           width=12288, topk=1024, poison=True)
    say("fused 4-row fp8", H, layout, B, req_rows)
    _fused_vs_two_calls(inp, f"fused mtp H{H} {layout} B{B}")


@pytest.mark.parametrize("H", [1, 2, 4])
@pytest.mark.parametrize("B", [16, 64, 3])
def test_fused_selection_shapes(H, B):
    """Ragged visible counts from a few columns to many chunks: rows that fit in
    k, short rows whose lists hold fewer than k keys (full-row selection), rows
    near 3k..8k (many chunks reach the threshold: their other columns are added),
    long rows; several rows per lane (H < 4), the per-column gather (B = 3),
    weights, and a visible count past the table (the full-row selection)."""
    k = 2048
    ctx = [0, 5, k, k + 1, 3000, 5000, 6500, 8200, 12000, 16001, 20000, 24100, 30000, 2 * k + 7, 9999, 15000]
    R = len(ctx)
    # the width runs past the table (columns 30,000+ of every row are -inf)
    inp = qsa_inputs.build(name="fused shapes", seed=40 + H + B, req_rows=[4] * (R // 4), ctx_rows=ctx,
                           num_heads=H, block_size=B, weights=True, topk=k, width=32768)
    say("fused shapes", H, B)
    _fused_vs_two_calls(inp, f"fused H{H} B{B}")
    # rows asking for more columns than the table holds (their selection reaches
    # the -inf columns past it), and past the width
    inp.ctx_lens = inp.ctx_lens.copy()
    inp.ctx_lens[11] = inp.width + 500
    inp.ctx_lens[12] = int(inp.max_blocks * inp.block_size) + 10
    _fused_vs_two_calls(inp, f"fused H{H} B{B} ctx past the table")


@pytest.mark.parametrize("kind", ["ties", "sorted", "spike"])
def test_fused_selection_adversarial_scores(kind):
    """Scores built to defeat the chunk lists: many equal scores (tie groups
    wider than the exact-ranking wave), keys ordered so that the largest scores
    crowd a few chunks (every list saturated), and one chunk holding far more
    than 16 of the row's top columns."""
    k = 2048
    ctx = [24000, 30000, 18000, 9000, 24000, 30000, 18000, 9000]
    inp = qsa_inputs.build(name="fused adv", seed=90, req_rows=[4, 4], ctx_rows=ctx, num_heads=4, block_size=16,
                           topk=k)
    B, D = inp.block_size, inp.head_dim
    kc = inp.kcache.copy()
    if kind == "ties":
        # keys from a handful of patterns: many columns score exactly alike
        pats = kc[:5].copy()
        kc[:] = pats[np.arange(kc.shape[0]) % 5]
    elif kind == "sorted":
        # scale each key by its position in the request: scores grow with the column
        for req in range(inp.num_reqs):
            for c in range(int(inp.kv_lens[req])):
                blk = inp.block_table[req, c // B]
                f = np.float32(0.2 + 3.0 * c / 30000.0)
                kc[blk, c % B] = qsa_inputs.f32_to_bf16_bits(
                    (kc[blk, c % B].astype(np.uint32) << 16).view(np.float32) * f)
    else:
        # columns 640..1279 of every request get keys 8x larger
        for req in range(inp.num_reqs):
            for c in range(640, 1280):
                blk = inp.block_table[req, c // B]
                kc[blk, c % B] = qsa_inputs.f32_to_bf16_bits(
                    (kc[blk, c % B].astype(np.uint32) << 16).view(np.float32) * np.float32(8.0))
    inp.kcache = kc
    say("fused adversarial", kind)
    _fused_vs_two_calls(inp, f"fused {kind}")


def test_fused_selection_without_workspace_and_in_a_graph():
    """No workspace: the same results without fusion.  Captured in a HIP graph:
    replays equal the eager call bit for bit, with other calls between them."""
    m = qsa()
    inp = qsa_inputs.make_config("decode_verify")
    other = qsa_inputs.make_config("decode_verify", seed=55)
    say("fused no workspace / graph")
    _fused_vs_two_calls(inp, "fused no workspace", workspace=None)
    dev, dev2 = to_device(inp), to_device(other)
    s = torch.cuda.Stream()
    out = torch.empty((inp.num_rows, inp.width), dtype=torch.float32, device="cuda")
    idx = torch.empty((inp.num_rows, inp.topk), dtype=torch.int32, device="cuda")
    out2 = torch.empty((other.num_rows, other.width), dtype=torch.float32, device="cuda")
    idx2 = torch.empty((other.num_rows, other.topk), dtype=torch.int32, device="cuda")
    call = m.PreparedLogitsTopk(dev.q, dev.kcache, dev.block_table, dev.ctx_lens, dev.row_to_req, out, idx,
                                k=inp.topk, width=inp.width, block_size=inp.block_size, stream=s)
    call2 = m.PreparedLogitsTopk(dev2.q, dev2.kcache, dev2.block_table, dev2.ctx_lens, dev2.row_to_req, out2, idx2,
                                 k=other.topk, width=other.width, block_size=other.block_size, stream=s)
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    ref, ref_idx = out.clone(), idx.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(idx, ref_idx), f"replay {r}"
        with torch.cuda.stream(s):
            call2()
        torch.cuda.synchronize()


def test_fused_selection_widest_rows():
    """Rows of up to 69,632 columns (two candidate lists per resolve thread)."""
    ctx = [69632, 69000, 65600, 40000, 66000, 2049, 69632, 50000]
    inp = qsa_inputs.build(name="fused wide", seed=97, req_rows=[4, 4], ctx_rows=ctx, num_heads=4, block_size=64,
                           topk=2048, width=69632)
    say("fused widest rows")
    _fused_vs_two_calls(inp, "fused wide")
