"""Pins for the CPU oracle: each one ties it to something other than itself.

Every ``pin_*`` takes the loaded oracle library (so the mutation harness can
run the same pins against a deliberately broken build) and raises
``AssertionError`` when the oracle disagrees with:

* a library routine (torch's bfloat16 / float8_e4m3fn widening, numpy matmul,
  numpy lexsort),
* a closed form (one-hot queries read a key element back; non-negative inputs
  make the ReLU the identity so the score is a GEMV),
* an invariant the pages state (zero-padded heads add 0: sglang PR #48649,
  Accuracy Tests; columns past the visible count are exactly -inf: ROCm/aiter
  PR #4221 test gate; results do not depend on where blocks sit in the pool),
* brute force over all subsets (selection), or
* a hand-worked example stored under tests/golden/.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

import oracle
import qsa_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# helpers (test side; library routines only)
# ----------------------------------------------------------------------------

def lib_bf16(bits: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def lib_e4m3fn(codes: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def lib_fp16(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def enc(dtype, values) -> np.ndarray:
    """float32 values -> the input encoding of dtype (library / numpy casts)."""
    if dtype == "bf16":
        return bf16(values)
    if dtype == "fp16":
        return qsa_inputs.f32_to_fp16_bits(values)
    return qsa_inputs.f32_to_e4m3fn_codes(np.asarray(values, dtype=np.float32))


def bf16(values) -> np.ndarray:
    return qsa_inputs.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


def identity_table(inp: qsa_inputs.PagedInputs) -> np.ndarray:
    """Rewrite the block table so request i owns consecutive pool blocks; return
    each request's first block."""
    B = inp.block_size
    starts = []
    pos = 0
    for i in range(inp.num_reqs):
        nb = int((inp.kv_lens[i] + B - 1) // B)
        inp.block_table[i, :nb] = np.arange(pos, pos + nb, dtype=np.int32)
        starts.append(pos)
        pos += nb
    return np.asarray(starts)


def contiguous_keys_f64(inp, starts) -> list:
    """Per request, its keys as a contiguous float64 [kv_len, D] array decoded by
    library routines (only valid after identity_table)."""
    B, D = inp.block_size, inp.head_dim
    out = []
    for i in range(inp.num_reqs):
        n = int(inp.kv_lens[i])
        s0 = int(starts[i]) * B
        if inp.dtype in ("bf16", "fp16"):
            flat = inp.kcache.reshape(-1, D)
            out.append((lib_bf16 if inp.dtype == "bf16" else lib_fp16)(flat[s0:s0 + n]))
        elif inp.layout == "paged":
            flat = inp.kcache.reshape(-1, D)
            sc = inp.kscale.reshape(-1).astype(np.float64) if inp.kscale is not None else None
            k = lib_e4m3fn(flat[s0:s0 + n])
            out.append(k if sc is None else k * sc[s0:s0 + n, None])
        else:
            nbk = inp.kcache.shape[0]
            keys = inp.kcache[:, : B * D].reshape(nbk * B, D)
            sc = inp.kcache[:, B * D:].copy().view("<f4").reshape(nbk * B).astype(np.float64)
            out.append(lib_e4m3fn(keys[s0:s0 + n]) * sc[s0:s0 + n, None])
    return out


def small(seed=11, dtype="bf16", layout="paged", H=4, B=16, req_rows=(2, 3), ctx=None,
          weights=False, **kw):
    if ctx is None:
        ctx = [37, 37, 50, 45, 50][: sum(req_rows)]
    return qsa_inputs.build(name="pin", seed=seed, req_rows=list(req_rows), ctx_rows=ctx,
                            num_heads=H, block_size=B, dtype=dtype, layout=layout,
                            weights=weights, **kw)


def visible(lg: np.ndarray, inp) -> list:
    ce = inp.ctx_eff()
    return [lg[r, : ce[r]] for r in range(inp.num_rows)]


# ----------------------------------------------------------------------------
# element decoders
# ----------------------------------------------------------------------------

def pin_e4m3fn_matches_library(lib):
    codes = np.arange(256, dtype=np.uint8)
    mine = np.array([lib.ora_e4m3fn_to_double(int(c)) for c in codes])
    ref = lib_e4m3fn(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def pin_e4m3fn_spec_points(lib):
    # OCP 8-bit FP spec, E4M3: bias 7, max normal S.1111.110 = 448,
    # min normal 2^-6, min subnormal 2^-9, S.1111.111 = NaN.
    f = lib.ora_e4m3fn_to_double
    assert f(0x38) == 1.0 and f(0xB8) == -1.0
    assert f(0x7E) == 448.0 and f(0xFE) == -448.0
    assert f(0x08) == 2.0 ** -6 and f(0x01) == 2.0 ** -9 and f(0x07) == 7 * 2.0 ** -9
    assert f(0x40) == 2.0 and f(0x3C) == 1.5
    assert np.isnan(f(0x7F)) and np.isnan(f(0xFF))
    assert f(0x00) == 0.0 and np.signbit(f(0x80))


def pin_bf16_matches_library(lib):
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=4096).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite patterns
    mine = np.array([lib.ora_bf16_to_double(int(b)) for b in bits])
    assert np.array_equal(mine, lib_bf16(bits))


def pin_fp16_matches_library(lib):
    """Every one of the 65,536 binary16 codes against numpy's float16 -> float64."""
    codes = np.arange(1 << 16, dtype=np.uint16)
    mine = np.array([lib.ora_fp16_to_double(int(c)) for c in codes])
    ref = lib_fp16(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def pin_fp16_spec_points(lib):
    # IEEE 754 binary16: bias 15, max 65504, min normal 2^-14, min subnormal 2^-24
    f = lib.ora_fp16_to_double
    assert f(0x3C00) == 1.0 and f(0xC000) == -2.0 and f(0x3555) == 1365 / 4096
    assert f(0x7BFF) == 65504.0 and f(0x0400) == 2.0 ** -14
    assert f(0x0001) == 2.0 ** -24 and f(0x03FF) == 1023 * 2.0 ** -24
    assert f(0x7C00) == np.inf and f(0xFC00) == -np.inf and np.isnan(f(0x7E00))
    assert f(0x0000) == 0.0 and np.signbit(f(0x8000))


# ----------------------------------------------------------------------------
# scoring
# ----------------------------------------------------------------------------

def pin_one_hot_closed_form(lib):
    """q[r,h] = a_h * e_{j_h}: head h's dot is a_h * k[col, j_h]; the logit is
    sum_h w_h * max(a_h * k[col, j_h], 0).  Signs of a_h differ between heads,
    so a ReLU applied after the head sum (or none) changes the value."""
    for dtype, layout in (("bf16", "paged"), ("fp16", "paged"), ("fp8", "paged"), ("fp8", "copacked")):
        inp = small(seed=21, dtype=dtype, layout=layout, H=4, B=16, weights=True)
        starts = identity_table(inp)
        keys = contiguous_keys_f64(inp, starts)
        R, H, D = inp.q.shape
        j = np.array([[3, 77, 127, 0], [64, 5, 9, 120], [1, 2, 3, 4], [100, 50, 25, 12],
                      [7, 7, 90, 33]])[:R]
        a = np.array([[1.0, -1.0, 2.0, -0.5], [-2.0, 1.0, 0.5, 1.0], [1.0, 1.0, -1.0, -1.0],
                      [0.5, -2.0, 1.0, 1.0], [-1.0, -1.0, 1.0, 2.0]])[:R]
        qf = np.zeros((R, H, D), dtype=np.float32)
        for r in range(R):
            for h in range(H):
                qf[r, h, j[r, h]] = a[r, h]
        inp.q = enc(dtype, qf)
        lg = oracle.paged_logits(inp, lib=lib)
        wv = inp.w.astype(np.float64)
        for r in range(R):
            req = inp.row_to_req[r]
            n = int(inp.ctx_eff()[r])
            k = keys[req][:n]
            exp = np.zeros(n)
            for h in range(H):
                exp += wv[r, h] * np.maximum(a[r, h] * k[:, j[r, h]], 0.0)
            assert np.allclose(lg[r, :n], exp, rtol=1e-15, atol=0), (dtype, layout, r)


def pin_gemv_nonnegative(lib):
    """With q >= 0 and k >= 0 every dot is >= 0, so the ReLU is the identity and
    sum_h w_h (q_h . k) = (sum_h w_h q_h) . k: a matrix-vector product."""
    for dtype, layout, H, D in (("bf16", "paged", 1, 128), ("bf16", "paged", 4, 128), ("fp16", "paged", 4, 128),
                                ("fp8", "copacked", 8, 128), ("bf16", "paged", 4, 64), ("fp8", "copacked", 4, 64)):
        inp = small(seed=31, dtype=dtype, layout=layout, H=H, B=16, weights=(H > 1), head_dim=D)
        starts = identity_table(inp)
        if dtype in ("bf16", "fp16"):
            inp.kcache = inp.kcache & np.uint16(0x7FFF)
            inp.q = inp.q & np.uint16(0x7FFF)
            qd = (lib_bf16 if dtype == "bf16" else lib_fp16)(inp.q)
        else:
            B, D = inp.block_size, inp.head_dim
            inp.kcache[:, : B * D] &= np.uint8(0x7F)
            inp.q = inp.q & np.uint8(0x7F)
            qd = lib_e4m3fn(inp.q)
        keys = contiguous_keys_f64(inp, starts)
        lg = oracle.paged_logits(inp, lib=lib)
        wv = np.ones((inp.num_rows, H)) if inp.w is None else inp.w.astype(np.float64)
        for r in range(inp.num_rows):
            n = int(inp.ctx_eff()[r])
            qeff = (wv[r][:, None] * qd[r]).sum(axis=0)
            exp = keys[inp.row_to_req[r]][:n] @ qeff
            assert np.allclose(lg[r, :n], exp, rtol=1e-12, atol=1e-12), (dtype, H, r)


def pin_relu_is_per_head(lib):
    """Head 0 scores +k[col, j] and head 1 scores -k[col, j]: a per-head ReLU gives
    |k[col, j]|, a ReLU after the sum would give 0."""
    inp = small(seed=41, H=2, req_rows=(1,), ctx=[40])
    starts = identity_table(inp)
    keys = contiguous_keys_f64(inp, starts)[0]
    qf = np.zeros((1, 2, 128), dtype=np.float32)
    qf[0, 0, 17] = 1.0
    qf[0, 1, 17] = -1.0
    inp.q = bf16(qf)
    lg = oracle.paged_logits(inp, lib=lib)
    assert np.array_equal(lg[0, :40], np.abs(keys[:40, 17]))


def pin_zero_heads_add_zero(lib):
    """sglang PR #48649, Accuracy Tests: padded heads are zero, so they add 0."""
    for dtype, layout in (("bf16", "paged"), ("fp16", "paged"), ("fp8", "copacked")):
        base = small(seed=51, dtype=dtype, layout=layout, H=4, weights=True)
        lg4 = oracle.paged_logits(base, lib=lib)
        pad = small(seed=51, dtype=dtype, layout=layout, H=4, weights=True)
        R, H, D = pad.q.shape
        q16 = np.zeros((R, 16, D), dtype=pad.q.dtype)
        q16[:, :4] = pad.q
        w16 = np.random.default_rng(3).uniform(0, 1, (R, 16)).astype(np.float32)
        w16[:, :4] = pad.w
        pad.q, pad.w, pad.num_heads = q16, w16, 16
        lg16 = oracle.paged_logits(pad, lib=lib)
        assert np.array_equal(lg4, lg16)


def pin_all_negative_is_zero(lib):
    inp = small(seed=61, H=4, weights=True)
    inp.kcache = inp.kcache & np.uint16(0x7FFF)
    inp.q = inp.q | np.uint16(0x8000)
    lg = oracle.paged_logits(inp, lib=lib)
    for r, v in enumerate(visible(lg, inp)):
        assert np.all(v == 0.0), r


def pin_mask_exact(lib):
    """Columns [ctx_eff, width) are exactly -inf and [0, ctx_eff) finite, with
    ctx clamped to min(width, max_blocks * block_size)."""
    inp = small(seed=71, req_rows=(2, 3), ctx=[0, 1, 16, 17, 400], kv_lens=[1, 64],
                max_blocks=4, width=70)
    lg = oracle.paged_logits(inp, lib=lib)
    ce = [0, 1, 16, 17, 64]
    assert list(inp.ctx_eff()) == ce
    for r in range(inp.num_rows):
        assert np.all(np.isfinite(lg[r, : ce[r]])), r
        assert np.all(lg[r, ce[r]:] == -np.inf), r
        assert int(np.isneginf(lg[r]).sum()) == 70 - ce[r]
    # width below the table capacity: the visible range stops at the width
    inp3 = small(seed=73, req_rows=(1,), ctx=[50], kv_lens=[64], max_blocks=4, width=40)
    lg3 = oracle.paged_logits(inp3, lib=lib)
    assert lg3.shape == (1, 40) and np.all(np.isfinite(lg3))
    inp2 = small(seed=72, req_rows=(1,), ctx=[-5])
    lg2 = oracle.paged_logits(inp2, lib=lib)
    assert np.all(lg2 == -np.inf)


def pin_block_permutation_invariant(lib):
    """Moving blocks within the pool and rewriting the table is bitwise neutral."""
    for dtype, layout in (("bf16", "paged"), ("fp16", "paged"), ("fp8", "paged"), ("fp8", "copacked")):
        inp = small(seed=81, dtype=dtype, layout=layout, weights=True, pool=12)
        lg = oracle.paged_logits(inp, lib=lib)
        perm = np.random.default_rng(9).permutation(inp.num_blocks)
        inv = np.argsort(perm)
        moved = small(seed=81, dtype=dtype, layout=layout, weights=True, pool=12)
        moved.kcache = inp.kcache[inv]  # new slot p holds old block inv[p]
        if inp.kscale is not None:
            moved.kscale = inp.kscale[inv]
        moved.block_table = perm[inp.block_table].astype(np.int32)
        assert np.array_equal(lg, oracle.paged_logits(moved, lib=lib))


def pin_row_order_free(lib):
    """Rows need not be request-major: each row follows its own row_to_req."""
    inp = small(seed=91, req_rows=(3, 2), ctx=[30, 31, 32, 20, 21], shuffle_rows=True)
    lg = oracle.paged_logits(inp, lib=lib)
    starts = identity_table(inp)
    keys = contiguous_keys_f64(inp, starts)
    lg2 = oracle.paged_logits(inp, lib=lib)
    qd = lib_bf16(inp.q)
    for r in range(inp.num_rows):
        n = int(inp.ctx_eff()[r])
        dots = keys[inp.row_to_req[r]][:n] @ qd[r].T
        exp = np.maximum(dots, 0.0).sum(axis=1)
        assert np.allclose(lg2[r, :n], exp, rtol=1e-12, atol=1e-12)
    assert lg.shape == lg2.shape


def pin_scale_powers_of_two(lib):
    """A per-key scale 2^e multiplies that key's logit by exactly 2^e
    (ReLU(s x) = s ReLU(x) for s >= 0, exact for powers of two)."""
    for layout in ("paged", "copacked"):
        inp = small(seed=101, dtype="fp8", layout=layout, weights=True, fp8_scale=False)
        lg1 = oracle.paged_logits(inp, lib=lib)
        rng = np.random.default_rng(4)
        B, D = inp.block_size, inp.head_dim
        e = rng.integers(-6, 7, size=(inp.num_blocks, B))
        s = np.ldexp(np.ones_like(e, dtype=np.float32), e).astype(np.float32)
        if layout == "paged":
            inp.kscale = s
        else:
            inp.kcache[:, B * D:] = s.astype("<f4").view(np.uint8).reshape(inp.num_blocks, 4 * B)
        lg2 = oracle.paged_logits(inp, lib=lib)
        for r in range(inp.num_rows):
            n = int(inp.ctx_eff()[r])
            req = inp.row_to_req[r]
            cols = np.arange(n)
            blk = inp.block_table[req, cols // B]
            ee = e[blk, cols % B]
            assert np.array_equal(lg2[r, :n], np.ldexp(lg1[r, :n], ee)), (layout, r)


def pin_unit_scale_layouts_agree(lib):
    """Paged fp8 without scales, with unit scales, and co-packed with unit scales
    give identical logits (they hold the same keys)."""
    a = small(seed=111, dtype="fp8", layout="paged", fp8_scale=False, weights=True)
    b = small(seed=111, dtype="fp8", layout="copacked", fp8_scale=False, weights=True)
    lga = oracle.paged_logits(a, lib=lib)
    a.kscale = None
    lgn = oracle.paged_logits(a, lib=lib)
    lgb = oracle.paged_logits(b, lib=lib)
    assert np.array_equal(lga, lgn) and np.array_equal(lga, lgb)


def pin_preshuffled_layout_equals_block_flat(lib):
    """ROCm/aiter PR #4221, preshuffle commit: only the intra-block key-byte
    offset changes, so the same keys in the preshuffled co-packed layout must
    give bitwise the same logits as in the block-flat one.  The generator's
    shuffle is also checked against the stated offset of byte d of slot s."""
    for H, B in ((4, 16), (64, 64), (16, 48)):
        flat = small(seed=121, dtype="fp8", layout="copacked", H=H, B=B, weights=True)
        shuf = small(seed=121, dtype="fp8", layout="copacked_shuffled", H=H, B=B, weights=True)
        D = flat.head_dim
        keys = flat.kcache[:, : B * D].reshape(-1, B, D)
        sec = shuf.kcache[:, : B * D]
        s_ = np.arange(B)[:, None]
        d_ = np.arange(D)[None, :]
        at = (s_ // 16) * 16 * D + (d_ // 16) * 256 + (s_ % 16) * 16 + d_ % 16
        assert np.array_equal(sec[:, at], keys)
        assert np.array_equal(shuf.kcache[:, B * D:], flat.kcache[:, B * D:])
        assert np.array_equal(oracle.paged_logits(flat, lib=lib), oracle.paged_logits(shuf, lib=lib))


def pin_weights_select_heads(lib):
    """w = e_h reduces the score to head h alone, i.e. the H = 1 problem on q[:, h]."""
    inp = small(seed=121, H=4, weights=True)
    for h in range(4):
        w = np.zeros_like(inp.w)
        w[:, h] = 1.0
        inp.w = w
        lg = oracle.paged_logits(inp, lib=lib)
        one = small(seed=121, H=4, weights=True)
        one.q = np.ascontiguousarray(one.q[:, h:h + 1, :])
        one.w, one.num_heads = None, 1
        assert np.array_equal(lg, oracle.paged_logits(one, lib=lib)), h


def pin_golden_hand_example(lib):
    """tests/golden/hand_example.json: a worked example computed by hand."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    D, H, B = g["head_dim"], g["num_heads"], g["block_size"]
    q = np.zeros((1, H, D), dtype=np.float32)
    for h, entries in enumerate(g["q_sparse"]):
        for d, v in entries:
            q[0, h, d] = v
    nb = len(g["pool_keys_sparse"])
    k = np.zeros((nb, B, D), dtype=np.float32)
    for blk, slots in enumerate(g["pool_keys_sparse"]):
        for slot, entries in enumerate(slots):
            for d, v in entries:
                k[blk, slot, d] = v
    inp = qsa_inputs.PagedInputs(
        name="hand", dtype="bf16", layout="paged", num_heads=H, head_dim=D, block_size=B,
        max_blocks=len(g["block_table"]), width=g["width"], topk=g["topk"], q=bf16(q),
        w=np.asarray([g["w"]], dtype=np.float32), kcache=bf16(k), kscale=None,
        block_table=np.asarray([g["block_table"]], dtype=np.int32),
        ctx_lens=np.asarray([g["ctx"]], dtype=np.int32), row_to_req=np.zeros(1, np.int32),
        kv_lens=np.asarray([g["ctx"]]))
    lg = oracle.paged_logits(inp, lib=lib)
    exp = np.array([(-np.inf if v is None else v) for v in g["expected_logits"]])
    assert np.array_equal(lg[0], exp), (lg[0], exp)
    tk = oracle.topk(lg.astype(np.float32), inp.ctx_lens, g["topk"], lib=lib)
    assert sorted(tk[0].tolist()) == sorted(g["expected_topk"])


# ----------------------------------------------------------------------------
# selection
# ----------------------------------------------------------------------------

def _valid_selection(v, sel, n):
    """The defining property: every kept column beats every dropped one, where a
    tie goes to the lower column."""
    s = set(sel)
    for i in s:
        for j in range(n):
            if j in s:
                continue
            if not (v[i] > v[j] or (v[i] == v[j] and i < j)):
                return False
    return True


def pin_topk_bruteforce(lib):
    rng = np.random.default_rng(7)
    for trial in range(60):
        n = int(rng.integers(0, 8))
        W = n + int(rng.integers(0, 3))
        k = int(rng.integers(1, 10))
        vals = rng.choice(np.array([-2.0, -0.0, 0.0, 1.0, 1.0, 3.5, -np.inf], np.float32), size=W)
        vals[n:] = -np.inf
        got = oracle.topk(vals[None, :], [n], k, lib=lib)[0]
        take = min(k, n)
        assert np.all(got[take:] == -1)
        matches = [c for c in itertools.combinations(range(n), take)
                   if _valid_selection(vals, c, n)]
        assert len(matches) == 1
        assert sorted(got[:take].tolist()) == list(matches[0]), (trial, vals, k)


def pin_topk_vs_lexsort(lib):
    rng = np.random.default_rng(8)
    R, W = 6, 3000
    ctx = np.array([3000, 2500, 2048, 100, 2049, 0])
    for kind in ("normal", "ints", "relu"):
        x = qsa_inputs.make_logits(R, W, ctx, seed=int(rng.integers(1000)), kind=kind)
        got = oracle.topk(x, ctx, 2048, lib=lib)
        for r in range(R):
            n = int(ctx[r])
            v = x[r, :n].astype(np.float64) + 0.0  # -0.0 + 0.0 == +0.0
            order = np.lexsort((np.arange(n), -v))
            exp = order[: min(2048, n)]
            assert sorted(got[r][got[r] >= 0].tolist()) == sorted(exp.tolist()), (kind, r)
            assert np.count_nonzero(got[r] >= 0) == min(2048, n)


def pin_topk_special_rows(lib):
    W = 600
    ctx = [0, 5, 256, 257, 600]
    x = qsa_inputs.make_logits(5, W, ctx, seed=3, kind="const")
    got = oracle.topk(x, ctx, 256, lib=lib)
    assert np.all(got[0] == -1)
    assert sorted(got[1][:5].tolist()) == list(range(5)) and np.all(got[1][5:] == -1)
    for r in (2, 3, 4):  # all equal: the lowest columns win
        assert sorted(got[r].tolist()) == list(range(256))


def pin_topk_tail_ignored(lib):
    """vLLM PR #62589, Validation: with NaN past the visible count the selection is
    unchanged (top-k reads only [0, visible))."""
    ctx = [10, 3000, 1999]
    a = qsa_inputs.make_logits(3, 3000, ctx, seed=12, tail="neginf")
    b = qsa_inputs.make_logits(3, 3000, ctx, seed=12, tail="nan")
    assert np.array_equal(oracle.topk(a, ctx, 2048, lib=lib), oracle.topk(b, ctx, 2048, lib=lib))


def pin_topk_signed_zero_ties(lib):
    x = np.array([[-0.0, 0.0, -0.0, 0.0, 1.0, -1.0]], dtype=np.float32)
    got = oracle.topk(x, [6], 3, lib=lib)[0]
    assert sorted(got.tolist()) == [0, 1, 4]


def pin_topk_rejects_visible_nan(lib):
    x = np.array([[1.0, np.nan, 2.0]], dtype=np.float32)
    try:
        oracle.topk(x, [3], 2, lib=lib)
    except oracle.OracleError:
        return
    raise AssertionError("NaN inside the visible range was accepted")


def pin_topk_row_starts_shift_invariant(lib):
    """A row's candidates placed at column s of a wider buffer, with row start s,
    select the same offsets as the same values at column 0 without starts
    (sglang PR #48649 test body: per-row starts and lengths); the columns in
    front of the start and past its end are never read (NaN there)."""
    rng = np.random.default_rng(21)
    W = 700
    for kind in ("normal", "ints", "const", "relu"):
        R = 8
        n = rng.integers(0, 300, size=R)
        s = rng.integers(0, W - 300, size=R)
        s[:3] = [0, 1, 3]  # aligned and unaligned starts
        base = qsa_inputs.make_logits(R, 300, n, seed=int(rng.integers(1000)), kind=kind)
        wide = np.full((R, W), np.nan, dtype=np.float32)
        for r in range(R):
            wide[r, s[r]:s[r] + n[r]] = base[r, :n[r]]
        for k in (1, 17, 256):
            want = oracle.topk(base, n, k, lib=lib)
            got = oracle.topk(wide, n, k, lib=lib, row_starts=s)
            assert np.array_equal(got, want), (kind, k)
            assert np.array_equal(oracle.topk(base, n, k, lib=lib, row_starts=np.zeros(R, np.int32)), want)


def pin_topk_row_starts_bruteforce(lib):
    """Tiny rows with starts: the unique valid selection of the window
    [s, s + n), reported as offsets from s."""
    rng = np.random.default_rng(22)
    for trial in range(60):
        W = int(rng.integers(1, 10))
        s = int(rng.integers(0, W + 1))
        n = int(rng.integers(0, W - s + 1))
        k = int(rng.integers(1, 8))
        vals = rng.choice(np.array([-2.0, -0.0, 0.0, 1.0, 1.0, 3.5, -np.inf], np.float32), size=W)
        got = oracle.topk(vals[None, :], [n], k, lib=lib, row_starts=[s])[0]
        win = vals[s:s + n]
        take = min(k, n)
        assert np.all(got[take:] == -1)
        matches = [c for c in itertools.combinations(range(n), take) if _valid_selection(win, c, n)]
        assert len(matches) == 1
        assert sorted(got[:take].tolist()) == list(matches[0]), (trial, vals, s, n, k)


def pin_topk_row_starts_clamped(lib):
    """Starts clamp to [0, width] and lengths to what is left of the row."""
    W = 50
    x = np.arange(W, dtype=np.float32)[None, :].repeat(4, axis=0)
    got = oracle.topk(x, [10, 10, 100, 5], 8, lib=lib, row_starts=[60, -7, 45, 50])
    assert np.all(got[0] == -1)                                       # start past the width: empty
    assert sorted(got[1].tolist()) == list(range(2, 10))              # start -7 -> 0: columns 2..9
    assert sorted(got[2][got[2] >= 0].tolist()) == [0, 1, 2, 3, 4]    # 45 + 100 -> 5 columns left
    assert np.count_nonzero(got[2] >= 0) == 5
    assert np.all(got[3] == -1)                                       # start at the width: empty


def _golden(name):
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)) as f:
        return json.load(f)


def pin_expand_golden(lib):
    g = _golden("expand_example.json")
    got = oracle.expand(np.array(g["idx"], np.int32), g["ratio"], token_lens=g["token_lens"], lib=lib)
    assert got.tolist() == g["expected"]


def pin_expand_properties(lib):
    """For every slot: a token t is either -1 or lies in its column's group
    (t // ratio == column, t % ratio == position in the group); without a token
    bound every selected column yields its whole group; the number of tokens of
    a column with a bound L is min(ratio, max(0, L - column * ratio)); ratio 1
    without a bound returns the indices unchanged."""
    rng = np.random.default_rng(23)
    for ratio in (1, 2, 4, 7):
        R, k = 5, 9
        idx = np.full((R, k), -1, np.int32)
        for r in range(R):
            m = int(rng.integers(0, k + 1))
            idx[r, :m] = np.sort(rng.choice(200, size=m, replace=False))
        tl = rng.integers(0, 200 * ratio, size=R).astype(np.int32)
        for bound in (None, tl):
            got = oracle.expand(idx, ratio, token_lens=bound, lib=lib)
            assert got.shape == (R, k * ratio)
            g3 = got.reshape(R, k, ratio)
            for r in range(R):
                for p in range(k):
                    c = int(idx[r, p])
                    toks = g3[r, p]
                    live = toks[toks >= 0]
                    if c < 0:
                        assert live.size == 0
                        continue
                    for j, t in enumerate(toks):
                        if t >= 0:
                            assert t // ratio == c and t % ratio == j
                    want = ratio if bound is None else min(ratio, max(0, int(bound[r]) - c * ratio))
                    assert live.size == want, (ratio, r, p, c)
                    assert np.all(toks[:want] >= 0) and np.all(toks[want:] == -1)
        if ratio == 1:
            assert np.array_equal(oracle.expand(idx, 1, lib=lib), idx)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
