"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI
and compare it with the oracle under the gates the pages state.

Gates:
* bf16 logits: |g - o| <= 5e-5 + 5e-5 |o| elementwise (ROCm/ATOM PR #2651,
  Accuracy: rtol / atol 5e-5), and the -inf mask exact.
* fp16 logits: the same gate.  The pages state none for fp16 (vLLM PR #62589,
  Details, only says the dot runs in fp16 with fp32 accumulation); products of
  two fp16 values are exact in float32 as bf16 ones are, so both differ from
  the oracle only by the float32 accumulation order over the same sums.
* fp8 logits: calc_diff(g, o) < 1e-3 over visible entries and the -inf mask
  exact (ROCm/aiter PR #4221, test gate).  The pages do not define calc_diff; it
  is read as 1 - 2 sum(g o) / sum(g^2 + o^2), the usual meaning of the name.
  This is the contract.  A global similarity can hide a few wrong columns, so
  every element is also held to an allowance of L 2^-23 A with
  A = sum_h |w_h| s sum_d |q_hd k8_d| (all magnitudes) and L = max(D, 128) + H + 2
  units.  L is empirical, not derived: the order and precision in which the
  gfx950 fp8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) sums its 128 products are
  not documented, and at D = 64 one element was 91.8 units off: more than
  the D + H + 2 units that a sequential float32 sum of the 64 products plus the
  head sum, weight and scale roundings could reach for the head counts tested.
  The largest observed units per (D, H) are printed by every fp8 comparison
  ("[fp8-units]") and recorded with the margin kept.
* top-k on identical float32 logits: exact set equality (the tie rule makes the
  answer unique).
* top-k end to end: the sets may differ only among near-ties of the oracle's
  k-th score (vLLM PR #62589, MI300X comment: a 1-ulp accumulation difference
  flips picks at exact ties): a column c outside the common part needs
  |o[c] - kth| <= tol[c] + max tol over the differing columns, with tol the
  elementwise logit gate above (bf16/fp16) or allowance (fp8), because a swap of
  columns a and b needs |o[a] - o[b]| <= tol[a] + tol[b].
"""
from __future__ import annotations

import numpy as np

import oracle
import qsa_inputs
from qsa_inputs.device import to_device


def qsa():
    import paged_mqa_logits_block_amd as m
    return m


# largest observed fp8 error per (head_dim, heads), in units of 2^-23 A; the
# test session prints it at the end
FP8_UNITS = {}


def gpu_logits(inp, dev=None, out=None, stream=None):
    m = qsa()
    dev = dev or to_device(inp)
    return m.paged_logits(dev.q, dev.kcache, dev.block_table, dev.ctx_lens, dev.row_to_req,
                          width=dev.width, block_size=dev.block_size, w=dev.w, kscale=dev.kscale,
                          layout=dev.layout, out=out, stream=stream)


def gpu_topk(logits_t, ctx_t, k, width=None, workspace="auto", row_starts=None):
    """qsa_topk; workspace "auto" takes the split selection where the shape has
    one, None forces one workgroup per row."""
    return qsa().topk(logits_t, ctx_t, k, width=width, workspace=workspace, row_starts=row_starts)


TOPK_PATHS = {"split": "auto", "single": None}


def bf16_tol(o):
    return 5e-5 + 5e-5 * np.abs(o)


def fp8_magnitude(inp, rows, cols_per_row):
    """A = sum_h |w| s sum_d |q k8| for the given (row, cols), float64."""
    D, H, B = inp.head_dim, inp.num_heads, inp.block_size
    qa = np.abs(oracle.decode_e4m3fn(np.arange(256, dtype=np.uint8)))
    qa = np.nan_to_num(qa)
    out = []
    for r, cols in zip(rows, cols_per_row):
        req = inp.row_to_req[r]
        qm = qa[inp.q[r]]  # [H, D]
        wv = np.ones(H) if inp.w is None else np.abs(inp.w[r].astype(np.float64))
        blk = inp.block_table[req, cols // B]
        slot = cols % B
        if inp.layout == "copacked_shuffled":
            d = np.arange(D)[None, :]
            at = (slot[:, None] // 16) * 16 * D + (d // 16) * 256 + (slot[:, None] % 16) * 16 + d % 16
            keys = inp.kcache[blk[:, None], at]
            sc = inp.kcache[:, B * D:].copy().view("<f4").reshape(-1, B)[blk, slot].astype(np.float64)
        elif inp.layout == "copacked":
            keys = inp.kcache[blk[:, None], slot[:, None] * D + np.arange(D)[None, :]]
            sc = inp.kcache[:, B * D:].copy().view("<f4").reshape(-1, B)[blk, slot].astype(np.float64)
        else:
            keys = inp.kcache[blk, slot]
            sc = (np.ones(len(cols)) if inp.kscale is None
                  else inp.kscale[blk, slot].astype(np.float64))
        km = qa[keys]  # [n, D]
        out.append((km @ qm.T) @ wv * np.abs(sc))
    return out


def fp8_units(inp):
    """The allowance L in units of 2^-23 A (empirical; see the module notes)."""
    return max(inp.head_dim, 128) + inp.num_heads + 2


def fp8_abs_bound(inp, rows, cols_per_row):
    """L 2^-23 A per element for the given (row, cols)."""
    L = fp8_units(inp) * 2.0 ** -23
    return [L * A for A in fp8_magnitude(inp, rows, cols_per_row)]


def calc_diff(g, o):
    g = g.astype(np.float64)
    o = o.astype(np.float64)
    den = np.sum(g * g + o * o)
    return 0.0 if den == 0 else 1.0 - 2.0 * np.sum(g * o) / den


def assert_logits_match(g, o, inp, rows=None, label=""):
    """g: float32 [n, W] from the GPU; o: float64 oracle [n, W] for the same rows.
    Returns each row's elementwise tolerance over its visible columns (the gate
    for bf16/fp16, the allowance for fp8), for the end-to-end top-k check."""
    rows = list(range(inp.num_rows)) if rows is None else list(rows)
    ce = inp.ctx_eff()
    assert g.shape == o.shape, (g.shape, o.shape)
    vis_g, vis_o = [], []
    for i, r in enumerate(rows):
        c = int(ce[r])
        gr, orow = g[i], o[i]
        assert np.all(orow[c:] == -np.inf)
        bad_mask = np.nonzero(gr[c:] != -np.inf)[0]
        assert bad_mask.size == 0, f"{label} row {r}: {bad_mask.size} columns past ctx {c} not -inf (first {c + bad_mask[0]})"
        assert np.all(np.isfinite(gr[:c])), f"{label} row {r}: non-finite visible logits"
        vis_g.append(gr[:c])
        vis_o.append(orow[:c])
    tols = []
    if inp.dtype in ("bf16", "fp16"):
        for i, r in enumerate(rows):
            d = np.abs(vis_g[i].astype(np.float64) - vis_o[i])
            tol = bf16_tol(vis_o[i])
            tols.append(tol)
            if d.size:
                j = int(np.argmax(d - tol))
                assert np.all(d <= tol), (f"{label} row {r} col {j}: gpu {vis_g[i][j]!r} oracle {vis_o[i][j]!r} "
                                          f"|d| {d[j]:.3g} > tol {tol[j]:.3g}")
    else:
        gg = np.concatenate(vis_g) if vis_g else np.zeros(0)
        oo = np.concatenate(vis_o) if vis_o else np.zeros(0)
        cd = calc_diff(gg, oo)
        assert cd < 1e-3, f"{label} calc_diff {cd}"
        mags = fp8_magnitude(inp, rows, [np.arange(int(ce[r])) for r in rows])
        L = fp8_units(inp)
        worst = 0.0
        for i, r in enumerate(rows):
            d = np.abs(vis_g[i].astype(np.float64) - vis_o[i])
            bound = L * 2.0 ** -23 * mags[i]
            tols.append(bound)
            if d.size:
                nz = mags[i] > 0
                if np.any(nz):
                    worst = max(worst, float(np.max(d[nz] / (2.0 ** -23 * mags[i][nz]))))
                j = int(np.argmax(d - bound))
                assert np.all(d <= bound + 1e-30), (
                    f"{label} row {r} col {j}: gpu {vis_g[i][j]!r} oracle {vis_o[i][j]!r} bound {bound[j]:.3g}")
        key = (inp.head_dim, inp.num_heads)
        FP8_UNITS[key] = max(FP8_UNITS.get(key, 0.0), worst)
    return tols


def assert_topk_exact(gi, oi, label=""):
    """Same logits on both sides: identical selections (as sets; -1 padding equal)."""
    assert gi.shape == oi.shape
    for r in range(gi.shape[0]):
        gs = np.sort(gi[r])
        os_ = np.sort(oi[r])
        assert np.array_equal(gs, os_), f"{label} row {r}: sets differ ({np.setdiff1d(gs, os_)[:5]} vs {np.setdiff1d(os_, gs)[:5]})"


def assert_topk_banded(gi, oi, o_logits, tols, label=""):
    """End to end: sets agree except among near-ties of the oracle's k-th score.
    tols[i]: row i's elementwise tolerance over its visible columns (as returned
    by assert_logits_match)."""
    for r in range(gi.shape[0]):
        gset = set(int(x) for x in gi[r] if x >= 0)
        oset = set(int(x) for x in oi[r] if x >= 0)
        assert len(gset) == len(oset) == int(np.sum(gi[r] >= 0)), f"{label} row {r}: sizes"
        if gset == oset:
            continue
        diff = sorted(gset ^ oset)
        kth = min(o_logits[r][list(oset)])
        tmax = max(float(tols[r][c]) for c in diff)
        # the oracle selects on its float32 rounding: half an ulp of slack
        slack = 2.0 ** -24 * abs(kth)
        for c in diff:
            band = float(tols[r][c]) + tmax + slack
            assert abs(o_logits[r][c] - kth) <= band, (
                f"{label} row {r}: column {c} (oracle {o_logits[r][c]!r}) differs but is not a near-tie of "
                f"{kth!r} (band {band:.3g})")
