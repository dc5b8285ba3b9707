"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and validates host arguments exactly as documented -- through the
*_check entry points, which make no HIP call."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsaidx.h")

m = pytest.importorskip("paged_mqa_logits_block_amd")

A = 0x10000  # a 16-byte aligned stand-in address (never dereferenced)


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"QSA_API\s+[\w\s\*]*?\b(qsa_\w+)\s*\(", text)))


def test_header_symbols_exported():
    syms = declared_symbols()
    assert set(syms) == set(m.EXPORTED), syms
    for s in syms:
        assert hasattr(m.lib, s), s
        assert ctypes.cast(getattr(m.lib, s), ctypes.c_void_p).value


def test_preshuffled_layout_validation():
    """The preshuffled co-packed layout: fp8 only, blocks of a multiple of 16,
    no separate scale array."""
    f8 = dict(q_dtype=m.FP8_E4M3FN, k_dtype=m.FP8_E4M3FN, kv_layout=m.KV_COPACKED_SHUFFLED)
    for B in (16, 48, 64, 400, 1024):
        assert chk(shape(block_size=B, **f8)) == m.OK
    for B in (1, 8, 100):
        assert chk(shape(block_size=B, **f8)) == m.E_UNSUPPORTED
    assert chk(shape(kv_layout=m.KV_COPACKED_SHUFFLED)) == m.E_UNSUPPORTED  # bf16
    assert chk(shape(block_size=64, **f8), ks=A) == m.E_INVALID
    assert chk(shape(kv_layout=3)) == m.E_INVALID


def test_fp16_validation():
    """fp16 keys: paged layout only, no per-key scale, q and k dtypes equal."""
    assert chk(shape(q_dtype=m.FP16, k_dtype=m.FP16, kv_layout=m.KV_COPACKED)) == m.E_UNSUPPORTED
    assert chk(shape(q_dtype=m.FP16, k_dtype=m.FP16), ks=A) == m.E_INVALID
    assert chk(shape(q_dtype=m.FP16, k_dtype=m.BF16)) == m.E_DTYPE
    assert chk(shape(q_dtype=m.BF16, k_dtype=m.FP16)) == m.E_DTYPE
    assert chk(shape(q_dtype=3, k_dtype=3)) == m.E_DTYPE


def test_version():
    assert m.version().startswith("qsaidx ")
    assert "gfx950" in m.version()


def shape(**kw):
    base = dict(num_rows=8, num_heads=4, head_dim=128, block_size=16, num_reqs=2, max_blocks=188,
                width=3008, q_dtype=m.BF16, k_dtype=m.BF16, kv_layout=m.KV_PAGED, num_blocks=256,
                out_stride=3008)
    base.update(kw)
    return m.LogitsShape(**base)


def chk(s, q=A, w=None, kc=A, ks=None, bt=A, ctx=A, r2r=A, out=A):
    return m.paged_logits_check(q, w, kc, ks, bt, ctx, r2r, out, s)


def test_logits_valid_configurations():
    assert chk(shape()) == m.OK
    assert chk(shape(q_dtype=m.FP8_E4M3FN, k_dtype=m.FP8_E4M3FN, kv_layout=m.KV_COPACKED,
                     num_heads=64, block_size=64)) == m.OK
    assert chk(shape(q_dtype=m.FP8_E4M3FN, k_dtype=m.FP8_E4M3FN), ks=A) == m.OK
    for H in (1, 2, 4, 8, 16, 32, 64):
        assert chk(shape(num_heads=H)) == m.OK
    # head dim 64 (per-tile kernel), every dtype
    assert chk(shape(head_dim=64)) == m.OK
    assert chk(shape(head_dim=64, q_dtype=m.FP8_E4M3FN, k_dtype=m.FP8_E4M3FN, kv_layout=m.KV_COPACKED_SHUFFLED)) == m.OK
    # fp16 q and keys, paged layout
    assert chk(shape(q_dtype=m.FP16, k_dtype=m.FP16)) == m.OK
    for B in (1, 3, 8, 16, 32, 48, 64, 100, 200, 400, 1024):
        assert chk(shape(block_size=B)) == m.OK
    # empty calls are valid whatever the pointers
    assert chk(shape(num_rows=0), q=None, bt=None, ctx=None, r2r=None, out=None, kc=None) == m.OK
    assert chk(shape(width=0, out_stride=1), out=A + 4) == m.OK
    assert m.last_error() == ""


@pytest.mark.parametrize("kw,ptrs,status", [
    (dict(num_rows=-1), {}, m.E_INVALID),
    (dict(width=-5), {}, m.E_INVALID),
    (dict(num_heads=0), {}, m.E_INVALID),
    (dict(block_size=0), {}, m.E_INVALID),
    (dict(num_blocks=0), {}, m.E_INVALID),
    (dict(out_stride=3000), {}, m.E_INVALID),
    ({}, dict(q=None), m.E_INVALID),
    ({}, dict(out=None), m.E_INVALID),
    ({}, dict(r2r=None), m.E_INVALID),
    (dict(q_dtype=m.FP8_E4M3FN), {}, m.E_DTYPE),  # mixed operand dtypes
    (dict(k_dtype=7, q_dtype=7), {}, m.E_DTYPE),
    (dict(kv_layout=9), {}, m.E_INVALID),
    (dict(kv_layout=m.KV_COPACKED), {}, m.E_UNSUPPORTED),  # co-packed bf16
    ({}, dict(ks=A), m.E_INVALID),  # a scale with bf16 keys
    (dict(head_dim=96), {}, m.E_UNSUPPORTED),
    (dict(head_dim=256), {}, m.E_UNSUPPORTED),
    (dict(num_heads=3), {}, m.E_UNSUPPORTED),
    (dict(num_heads=128), {}, m.E_UNSUPPORTED),
    (dict(block_size=2048), {}, m.E_UNSUPPORTED),
    (dict(block_size=1025), {}, m.E_UNSUPPORTED),
    (dict(width=(1 << 24) + 16, out_stride=(1 << 24) + 16), {}, m.E_RANGE),
    (dict(num_blocks=1 << 51), {}, m.E_RANGE),
    ({}, dict(q=A + 4), m.E_ALIGN),
    ({}, dict(kc=A + 8), m.E_ALIGN),
    ({}, dict(out=A + 4), m.E_ALIGN),
    (dict(out_stride=3010), {}, m.E_ALIGN),
])
def test_logits_rejections(kw, ptrs, status):
    st = chk(shape(**kw), **ptrs)
    assert st == status, (st, m.last_error())
    assert m.last_error()


def test_shape_null():
    assert m.lib.qsa_paged_logits_check(A, None, A, None, A, A, A, A, None) == m.E_INVALID


@pytest.mark.parametrize("args,status", [
    ((A, 3008, A, 8, 3008, 256, A), m.OK),
    ((A, 69632, A, 8, 69632, 2048, A), m.OK),
    ((A, 3008, A, 8, 3008, 1, A), m.OK),
    ((None, 16, None, 0, 16, 8, None), m.OK),
    ((A, 3008, A, -1, 3008, 256, A), m.E_INVALID),
    ((A, 3008, A, 8, -1, 256, A), m.E_INVALID),
    ((A, 3008, A, 8, 3008, 0, A), m.E_INVALID),
    ((A, 3000, A, 8, 3008, 256, A), m.E_INVALID),
    ((None, 3008, A, 8, 3008, 256, A), m.E_INVALID),
    ((A, 3008, A, 8, 3008, 256, None), m.E_INVALID),
    ((A, 3008, A, 8, 3008, 2049, A), m.E_UNSUPPORTED),
    ((A, 69636, A, 8, 69636, 256, A), m.E_UNSUPPORTED),
    ((A + 4, 3008, A, 8, 3008, 256, A), m.E_ALIGN),
    ((A, 3010, A, 8, 3008, 256, A), m.E_ALIGN),
])
def test_topk_validation(args, status):
    st = m.topk_check(*args)
    assert st == status, (st, m.last_error())


@pytest.mark.parametrize("rows,width,split", [
    (36, 29408, True), (64, 65600, True), (47, 32768, True), (48, 32769, True), (128, 32772, True),
    (15, 69632, True), (8, 3008, False), (36, 4096, False), (48, 32768, False), (64, 32768, False),
    (128, 8192, False), (129, 29408, False), (16384, 28672, False), (0, 29408, False),
])
def test_topk_workspace_size(rows, width, split):
    """Up to 47 rows of more than 4096 columns, or up to 128 rows wider than
    the register path's 32,768 columns, use the split selection (a workspace);
    other shapes use one workgroup per row (no workspace)."""
    nbytes = m.topk_workspace_bytes(rows, width, 2048)
    assert (nbytes > 0) == split, nbytes
    if split:  # counts, a 256-bucket histogram and <= 8192 member slots of 8 bytes per row
        assert nbytes <= rows * (17 * 8 + 17 * 1024 + 8192 * 8) + 256


def test_topk_workspace_validation():
    need = m.topk_workspace_bytes(36, 29408, 2048)
    base = (A, 29408, A, 36, 29408, 2048, A)
    assert m.topk_check(*base, None, 0) == m.OK                 # NULL: one workgroup per row
    assert m.topk_check(*base, A, need) == m.OK
    assert m.topk_check(*base, A, need - 1) == m.E_INVALID
    assert m.topk_check(*base, A + 8, need) == m.E_ALIGN
    # a shape that uses no workspace accepts any
    assert m.topk_check(A, 3008, A, 8, 3008, 256, A, A + 8, 0) == m.OK


def test_one_hip_runtime_in_process():
    """The binding must share torch's HIP runtime (streams and allocations are
    torch's); a second copy of libamdhip64 in the process breaks launches."""
    maps = open("/proc/self/maps").read().splitlines()
    libs = sorted({ln.split()[-1] for ln in maps if "libamdhip64" in ln})
    assert len(libs) == 1, libs


def test_expand_validation():
    """qsa_expand refuses bad sizes before any launch (no HIP call)."""
    L = m.lib
    assert L.qsa_expand(A, -1, 8, 4, None, A, None) == m.E_INVALID
    assert L.qsa_expand(A, 2, 0, 4, None, A, None) == m.E_INVALID
    assert L.qsa_expand(A, 2, 8, 0, None, A, None) == m.E_INVALID
    assert L.qsa_expand(A, 2, 1 << 22, 8, None, A, None) == m.E_RANGE
    assert L.qsa_expand(None, 2, 8, 4, None, A, None) == m.E_INVALID
    assert L.qsa_expand(A, 2, 8, 4, None, None, None) == m.E_INVALID
    assert L.qsa_expand(None, 0, 8, 4, None, None, None) == m.OK  # nothing to do, nothing launched


def test_topk_row_starts_need_no_host_check():
    """Row starts are device data (clamped by the kernels): a pointer or NULL
    validates the same."""
    base = (A, 3008, A, 8, 3008, 256, A, None, 0)
    assert m.topk_check(*base) == m.OK
    assert m.topk_check(*base, row_starts_ptr=A) == m.OK


def test_bench_topk_plan_matches_the_library():
    """bench.py names the top-k kernels it times from its own copy of the
    planner's rule; it agrees with the library's workspace query on every
    workload and at the rule's edges."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    class Shape:
        def __init__(self, num_rows, width):
            self.num_rows, self.width = num_rows, width

    # the edges, and the workloads' (rows, width): tiny, decode_verify (and its
    # fp16 and D = 64 forms), single_row_mixed, the fp8 4-row shapes, ragged
    # and prefill_chunk
    shapes = [Shape(r, w) for r in (1, 36, 47, 48, 64, 128, 129) for w in (4096, 4097, 32768, 32769, 65600)]
    shapes += [Shape(r, w) for r, w in ((8, 3008), (36, 29408), (64, 65600), (64, 32768), (63, 32768),
                                        (16384, 28672))]
    for s in shapes:
        split = m.topk_workspace_bytes(s.num_rows, s.width, 2048) > 0
        assert (bench.topk_plan(s) == "split") == split, (s.num_rows, s.width)
