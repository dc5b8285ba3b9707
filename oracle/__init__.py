"""CPU oracle for paged MQA-logits scoring and per-row top-k (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg.  The product path (``paged_mqa_logits_block_amd``)
never imports this package, and this package never imports the product path.

The arithmetic lives in ``qsa_oracle.c`` (float64, definition order); this
module only marshals numpy arrays.  See that file's header for the passages it
follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "qsa_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

GCC_CMD = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB, SRC, "-lm"]


def build_lib(src: str = SRC, out: str = LIB) -> str:
    cmd = list(GCC_CMD)
    cmd[cmd.index(LIB)] = out
    cmd[cmd.index(SRC)] = src
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: Optional[str] = None):
    """Load the oracle library (building it only when it is absent)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB
    if not os.path.exists(p):
        build_lib(out=p)
    lib = ctypes.CDLL(p)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.ora_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.ora_bf16_to_double.restype = ctypes.c_double
    lib.ora_fp16_to_double.argtypes = [ctypes.c_uint16]
    lib.ora_fp16_to_double.restype = ctypes.c_double
    lib.ora_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
    lib.ora_e4m3fn_to_double.restype = ctypes.c_double
    lib.ora_paged_logits.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, i32p, i32p, i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    lib.ora_paged_logits.restype = ctypes.c_int
    lib.ora_topk.argtypes = [ctypes.c_void_p, ctypes.c_int64, i32p, ctypes.c_void_p, ctypes.c_int,
                             ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    lib.ora_topk.restype = ctypes.c_int
    lib.ora_expand.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_void_p, ctypes.c_void_p]
    lib.ora_expand.restype = ctypes.c_int
    lib.ora_max_threads.argtypes = []
    lib.ora_max_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class OracleError(RuntimeError):
    pass


_GUARD = 64
_DTYPE_CODES = {"bf16": 0, "fp8": 1, "fp16": 2}
_LAYOUT_CODES = {"paged": 0, "copacked": 1, "copacked_shuffled": 2}
_SENTINEL = 1.2345e300


def decode_bf16(bits) -> np.ndarray:
    lib = load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.ora_bf16_to_double(int(v)) for v in b.ravel()]).reshape(b.shape)


def decode_fp16(bits) -> np.ndarray:
    lib = load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.ora_fp16_to_double(int(v)) for v in b.ravel()]).reshape(b.shape)


def decode_e4m3fn(codes) -> np.ndarray:
    lib = load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.ora_e4m3fn_to_double(int(v)) for v in c.ravel()]).reshape(c.shape)


def paged_logits(inp, rows: Optional[Sequence[int]] = None, threads: int = 0,
                 lib=None) -> np.ndarray:
    """float64 logits ``[len(rows) or R, width]`` for a ``qsa_inputs.PagedInputs``."""
    lib = lib or load()
    q = np.ascontiguousarray(inp.q)
    w = None if inp.w is None else np.ascontiguousarray(inp.w, dtype=np.float32)
    kc = np.ascontiguousarray(inp.kcache)
    ks = None if inp.kscale is None else np.ascontiguousarray(inp.kscale, dtype=np.float32)
    bt = np.ascontiguousarray(inp.block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(inp.ctx_lens, dtype=np.int32)
    r2r = np.ascontiguousarray(inp.row_to_req, dtype=np.int32)
    sel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n = inp.num_rows if sel is None else len(sel)
    # a sentinel tail after the last row catches any write past n * width
    buf = np.empty(n * inp.width + _GUARD, dtype=np.float64)
    buf[n * inp.width:] = _SENTINEL
    out = buf[: n * inp.width].reshape(n, inp.width)
    st = lib.ora_paged_logits(
        _ptr(q), _DTYPE_CODES[inp.dtype], _ptr(w), _ptr(kc),
        _LAYOUT_CODES[inp.layout], _ptr(ks), _i32(bt), _i32(ctx), _i32(r2r),
        inp.num_rows, inp.num_heads, inp.head_dim, inp.block_size, inp.num_reqs,
        inp.max_blocks, inp.num_blocks, inp.width, _ptr(sel), n, _ptr(out), threads)
    if st != 0:
        raise OracleError(f"ora_paged_logits status {st}")
    if not np.array_equal(buf[n * inp.width:], np.full(_GUARD, _SENTINEL)):
        raise OracleError("ora_paged_logits wrote past the end of its output")
    return out


def topk(logits: np.ndarray, ctx_lens, k: int, threads: int = 0, lib=None, row_starts=None) -> np.ndarray:
    """int32 ``[R, k]`` offsets from each row's start (0 without ``row_starts``);
    -1 past min(k, candidates)."""
    lib = lib or load()
    x = np.ascontiguousarray(logits, dtype=np.float32)
    R, W = x.shape
    ctx = np.ascontiguousarray(np.asarray(ctx_lens).reshape(R), dtype=np.int32)
    st = None if row_starts is None else np.ascontiguousarray(np.asarray(row_starts).reshape(R), dtype=np.int32)
    out = np.empty((R, k), dtype=np.int32)
    status = lib.ora_topk(_ptr(x), W, _i32(ctx), _ptr(st), R, W, int(k), _ptr(out), threads)
    if status != 0:
        raise OracleError(f"ora_topk status {status}")
    return out


def expand(idx: np.ndarray, ratio: int, token_lens=None, lib=None) -> np.ndarray:
    """int32 ``[R, k * ratio]`` tokens of the selected compressed columns."""
    lib = lib or load()
    i = np.ascontiguousarray(idx, dtype=np.int32)
    R, k = i.shape
    tl = None if token_lens is None else np.ascontiguousarray(np.asarray(token_lens).reshape(R), dtype=np.int32)
    out = np.empty((R, k * int(ratio)), dtype=np.int32)
    status = lib.ora_expand(_ptr(i), R, k, int(ratio), _ptr(tl), _ptr(out))
    if status != 0:
        raise OracleError(f"ora_expand status {status}")
    return out


def select(inp, rows: Optional[Sequence[int]] = None, threads: int = 0):
    """Oracle logits (float64), their float32 rounding, and the top-k on the latter."""
    lg = paged_logits(inp, rows=rows, threads=threads)
    lg32 = lg.astype(np.float32)
    ctx = inp.ctx_lens if rows is None else np.asarray(inp.ctx_lens)[np.asarray(rows)]
    return lg, lg32, topk(lg32, ctx, inp.topk, threads=threads)


def max_threads() -> int:
    return int(load().ora_max_threads())
