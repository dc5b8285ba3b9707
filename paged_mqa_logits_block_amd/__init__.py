"""Python binding of libqsaidx: paged MQA-logits scoring and per-row top-k on
MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/qsaidx.h``.  Tensors are torch
device tensors (torch is used for device memory and streams); calls are queued
on the current torch stream unless ``stream`` is given.  Importing this module
fails loudly when the compiled library is absent.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsaidx.so")

# qsa_status
OK, E_INVALID, E_DTYPE, E_UNSUPPORTED, E_RANGE, E_ALIGN, E_HIP = range(7)
STATUS_NAMES = {0: "QSA_OK", 1: "QSA_E_INVALID", 2: "QSA_E_DTYPE", 3: "QSA_E_UNSUPPORTED",
                4: "QSA_E_RANGE", 5: "QSA_E_ALIGN", 6: "QSA_E_HIP"}
# qsa_dtype / qsa_kv_layout
BF16, FP8_E4M3FN, FP16 = 0, 1, 2
KV_PAGED, KV_COPACKED, KV_COPACKED_SHUFFLED = 0, 1, 2

EXPORTED = ("qsa_paged_logits", "qsa_paged_logits_timed", "qsa_paged_logits_check", "qsa_topk",
            "qsa_topk_timed", "qsa_topk_check", "qsa_topk_workspace_bytes", "qsa_topk_noalloc",
            "qsa_paged_logits_topk", "qsa_paged_logits_topk_timed", "qsa_paged_logits_topk_workspace_bytes",
            "qsa_expand", "qsa_last_error", "qsa_version")


class QsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class LogitsShape(ctypes.Structure):
    _fields_ = [
        ("num_rows", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_reqs", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
        ("width", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
        ("k_dtype", ctypes.c_int32), ("kv_layout", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64), ("out_stride", ctypes.c_int64),
    ]


def _load():
    # torch ships its own HIP runtime under the same soname as /opt/rocm's.
    # Importing torch first makes libqsaidx bind to that one runtime, which
    # also owns the device allocations and stream handles passed in; loading
    # the library first would start a second runtime in the process.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32p, i64, i32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sp = ctypes.POINTER(LogitsShape)
    lib.qsa_paged_logits.argtypes = [vp, vp, vp, vp, i32p, i32p, i32p, vp, sp, vp]
    lib.qsa_paged_logits.restype = ctypes.c_int
    lib.qsa_paged_logits_timed.argtypes = [vp, vp, vp, vp, i32p, i32p, i32p, vp, sp, vp, vp, vp]
    lib.qsa_paged_logits_timed.restype = ctypes.c_int
    lib.qsa_paged_logits_check.argtypes = [vp, vp, vp, vp, i32p, i32p, i32p, vp, sp]
    lib.qsa_paged_logits_check.restype = ctypes.c_int
    lib.qsa_topk.argtypes = [vp, i64, i32p, i32p, i32, i32, i32, i32p, vp, i64, vp]
    lib.qsa_topk.restype = ctypes.c_int
    lib.qsa_topk_timed.argtypes = [vp, i64, i32p, i32p, i32, i32, i32, i32p, vp, i64, vp, vp, vp]
    lib.qsa_topk_timed.restype = ctypes.c_int
    lib.qsa_topk_check.argtypes = [vp, i64, i32p, i32p, i32, i32, i32, i32p, vp, i64]
    lib.qsa_topk_check.restype = ctypes.c_int
    lib.qsa_paged_logits_topk.argtypes = [vp, vp, vp, vp, i32p, i32p, i32p, vp, sp, i32, i32p, vp, i64, vp]
    lib.qsa_paged_logits_topk.restype = ctypes.c_int
    lib.qsa_paged_logits_topk_timed.argtypes = [vp, vp, vp, vp, i32p, i32p, i32p, vp, sp, i32, i32p, vp, i64, vp,
                                                vp, vp, vp]
    lib.qsa_paged_logits_topk_timed.restype = ctypes.c_int
    lib.qsa_paged_logits_topk_workspace_bytes.argtypes = [sp, i32]
    lib.qsa_paged_logits_topk_workspace_bytes.restype = ctypes.c_int64
    lib.qsa_topk_noalloc.argtypes = [vp, i64, i32p, i32p, i32, i32, i32, i32p, vp]
    lib.qsa_topk_noalloc.restype = ctypes.c_int
    lib.qsa_expand.argtypes = [i32p, i32, i32, i32, i32p, i32p, vp]
    lib.qsa_expand.restype = ctypes.c_int
    lib.qsa_topk_workspace_bytes.argtypes = [i32, i32, i32]
    lib.qsa_topk_workspace_bytes.restype = ctypes.c_int64
    lib.qsa_last_error.argtypes = []
    lib.qsa_last_error.restype = ctypes.c_char_p
    lib.qsa_version.argtypes = []
    lib.qsa_version.restype = ctypes.c_char_p
    return lib


lib = _load()


def version() -> str:
    return lib.qsa_version().decode()


def last_error() -> str:
    return lib.qsa_last_error().decode()


def _raise_on(status: int):
    if status != OK:
        raise QsaError(status, last_error())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP8_E4M3FN
    if t.dtype == torch.float16:
        return FP16
    raise QsaError(E_DTYPE, f"unsupported tensor dtype {t.dtype}")


def _require(cond: bool, msg: str):
    if not cond:
        raise QsaError(E_INVALID, msg)


def make_shape(q, kcache, block_table, *, width: int, block_size: int, layout: int = KV_PAGED,
               out_stride: Optional[int] = None, num_blocks: Optional[int] = None) -> LogitsShape:
    R, H, D = (int(x) for x in q.shape)
    return LogitsShape(
        num_rows=R, num_heads=H, head_dim=D, block_size=int(block_size),
        num_reqs=int(block_table.shape[0]), max_blocks=int(block_table.shape[1]),
        width=int(width), q_dtype=_dtype_code(q), k_dtype=_dtype_code(kcache),
        kv_layout=int(layout),
        num_blocks=int(kcache.shape[0] if num_blocks is None else num_blocks),
        out_stride=int(width if out_stride is None else out_stride))


def _event(e) -> Optional[int]:
    """hipEvent_t of a torch.cuda.Event (created on its first record)."""
    return None if e is None else int(e.cuda_event)


def paged_logits(q, kcache, block_table, ctx_lens, row_to_req, *, width: int, block_size: int,
                 w=None, kscale=None, layout: int = KV_PAGED, out=None, stream=None, events=None):
    """``qsa_paged_logits``: f32 logits ``[R, width]`` (or into ``out``, whose row
    stride may exceed ``width``).  See include/qsaidx.h for the contract.
    ``events=(start, stop)`` (recorded torch.cuda.Event objects) routes the call
    through ``qsa_paged_logits_timed``."""
    import torch
    for name, t in (("q", q), ("kcache", kcache), ("block_table", block_table),
                    ("ctx_lens", ctx_lens), ("row_to_req", row_to_req), ("w", w), ("kscale", kscale)):
        if t is not None:
            _require(t.is_cuda, f"{name} must be a device tensor")
            _require(t.is_contiguous(), f"{name} must be contiguous")
    _require(q.dim() == 3, "q must be [R, H, D]")
    for name, t in (("block_table", block_table), ("ctx_lens", ctx_lens), ("row_to_req", row_to_req)):
        _require(t.dtype == torch.int32, f"{name} must be int32")
    if w is not None:
        _require(w.dtype == torch.float32 and tuple(w.shape) == tuple(q.shape[:2]), "w must be f32 [R, H]")
    if kscale is not None:
        _require(kscale.dtype == torch.float32, "kscale must be f32")
    R = int(q.shape[0])
    _require(int(ctx_lens.numel()) == R and int(row_to_req.numel()) == R, "ctx_lens / row_to_req must have R entries")
    if out is None:
        # rows padded to a multiple of 4 floats (the ABI's out_stride rule);
        # the result is the [R, width] view
        out = torch.empty((R, (width + 3) & ~3), dtype=torch.float32, device=q.device)[:, :width]
    _require(out.dtype == torch.float32 and out.dim() == 2 and out.stride(1) == 1, "out must be f32 [R, >=width]")
    shape = make_shape(q, kcache, block_table, width=width, block_size=block_size, layout=layout,
                       out_stride=out.stride(0) if R > 0 else width)
    args = (_ptr(q), _ptr(w), _ptr(kcache), _ptr(kscale), _ptr(block_table), _ptr(ctx_lens),
            _ptr(row_to_req), _ptr(out), ctypes.byref(shape), _stream(stream))
    if events is None:
        st = lib.qsa_paged_logits(*args)
    else:
        st = lib.qsa_paged_logits_timed(*args, _event(events[0]), _event(events[1]))
    _raise_on(st)
    return out


def topk_workspace_bytes(num_rows: int, width: int, k: int) -> int:
    """``qsa_topk_workspace_bytes``: scratch bytes the split selection uses (0: none)."""
    return int(lib.qsa_topk_workspace_bytes(int(num_rows), int(width), int(k)))


def _torch_stream(stream):
    """The torch stream object for a `stream` argument (None: the current one)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _workspace(workspace, R: int, width: int, k: int, device, stream=None):
    """(tensor or None, pointer, bytes) for qsa_topk's workspace argument:
    "auto" allocates what the shape uses (nothing when it uses none), None
    passes NULL (one workgroup per row), a uint8 device tensor is passed as is.
    An "auto" workspace is marked as in use on the launch stream, so the caching
    allocator does not hand its memory to other work before the kernels that use
    it have run, even after the last Python reference is gone."""
    import torch
    if workspace is None:
        return None, None, 0
    if isinstance(workspace, str):
        _require(workspace == "auto", 'workspace must be "auto", None or a device tensor')
        nbytes = topk_workspace_bytes(R, width, k)
        if nbytes == 0:
            return None, None, 0
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        workspace.record_stream(_torch_stream(stream))
    _require(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous device tensor")
    return workspace, workspace.data_ptr(), int(workspace.numel() * workspace.element_size())


def _check_rows_i32(name, t, R):
    import torch
    _require(t.is_cuda and t.dtype == torch.int32 and t.is_contiguous() and int(t.numel()) == R,
             f"{name} must be a contiguous int32 device tensor with one entry per row")


def topk(logits, ctx_lens, k: int, *, width: Optional[int] = None, row_starts=None, out=None,
         workspace="auto", stream=None, events=None):
    """``qsa_topk``: int32 ``[R, k]`` selected offsets from each row's start
    (``row_starts``, default 0), ascending, -1 padded.
    ``workspace``: "auto" (allocate the scratch the shape uses), None (NULL:
    one workgroup per row) or a uint8 device tensor."""
    import torch
    _require(logits.is_cuda and ctx_lens.is_cuda, "logits and ctx_lens must be device tensors")
    _require(logits.dtype == torch.float32 and logits.dim() == 2 and logits.stride(1) == 1,
             "logits must be f32 [R, >=width] with unit column stride")
    _require(ctx_lens.dtype == torch.int32 and ctx_lens.is_contiguous(), "ctx_lens must be contiguous int32")
    R = int(logits.shape[0])
    if row_starts is not None:
        _check_rows_i32("row_starts", row_starts, R)
    width = int(logits.shape[1]) if width is None else int(width)
    if out is None:
        out = torch.empty((R, k), dtype=torch.int32, device=logits.device)
    _require(out.dtype == torch.int32 and out.is_contiguous() and tuple(out.shape) == (R, k),
             "out must be contiguous int32 [R, k]")
    stride = int(logits.stride(0)) if R > 0 else width
    ws, ws_ptr, ws_bytes = _workspace(workspace, R, width, k, logits.device, stream)
    args = (_ptr(logits), stride, _ptr(ctx_lens), _ptr(row_starts), R, width, int(k), _ptr(out), ws_ptr,
            ws_bytes, _stream(stream))
    if events is None:
        st = lib.qsa_topk(*args)
    else:
        st = lib.qsa_topk_timed(*args, _event(events[0]), _event(events[1]))
    _raise_on(st)
    return out


def topk_noalloc(logits, ctx_lens, k: int, *, width: Optional[int] = None, row_starts=None, out=None,
                 stream=None):
    """``qsa_topk_noalloc``: as ``topk`` with the library-held scratch instead of
    a workspace (the call allocates no device memory; ``out`` may be given so
    that nothing is allocated here either)."""
    import torch
    _require(logits.is_cuda and ctx_lens.is_cuda, "logits and ctx_lens must be device tensors")
    _require(logits.dtype == torch.float32 and logits.dim() == 2 and logits.stride(1) == 1,
             "logits must be f32 [R, >=width] with unit column stride")
    _require(ctx_lens.dtype == torch.int32 and ctx_lens.is_contiguous(), "ctx_lens must be contiguous int32")
    R = int(logits.shape[0])
    if row_starts is not None:
        _check_rows_i32("row_starts", row_starts, R)
    width = int(logits.shape[1]) if width is None else int(width)
    if out is None:
        out = torch.empty((R, k), dtype=torch.int32, device=logits.device)
    _require(out.dtype == torch.int32 and out.is_contiguous() and tuple(out.shape) == (R, k),
             "out must be contiguous int32 [R, k]")
    stride = int(logits.stride(0)) if R > 0 else width
    _raise_on(lib.qsa_topk_noalloc(_ptr(logits), stride, _ptr(ctx_lens), _ptr(row_starts), R, width, int(k),
                                   _ptr(out), _stream(stream)))
    return out


def expand(idx, ratio: int, *, token_lens=None, out=None, stream=None):
    """``qsa_expand``: int32 ``[R, k * ratio]`` tokens of the selected compressed
    columns (column c covers tokens c * ratio .. c * ratio + ratio - 1), -1 for
    padding and for tokens at or past ``token_lens``."""
    import torch
    _require(idx.is_cuda and idx.dtype == torch.int32 and idx.dim() == 2 and idx.is_contiguous(),
             "idx must be a contiguous int32 [R, k] device tensor")
    R, k = (int(x) for x in idx.shape)
    if token_lens is not None:
        _check_rows_i32("token_lens", token_lens, R)
    if out is None:
        out = torch.empty((R, k * int(ratio)), dtype=torch.int32, device=idx.device)
    _require(out.dtype == torch.int32 and out.is_contiguous() and tuple(out.shape) == (R, k * int(ratio)),
             "out must be contiguous int32 [R, k * ratio]")
    _raise_on(lib.qsa_expand(_ptr(idx), R, k, int(ratio), _ptr(token_lens), _ptr(out), _stream(stream)))
    return out


def paged_logits_check(q_ptr, w_ptr, kcache_ptr, kscale_ptr, bt_ptr, ctx_ptr, r2r_ptr, out_ptr,
                       shape: LogitsShape) -> int:
    """Host-side validation only (``qsa_paged_logits_check``); pointers are ints."""
    return lib.qsa_paged_logits_check(q_ptr, w_ptr, kcache_ptr, kscale_ptr, bt_ptr, ctx_ptr, r2r_ptr,
                                      out_ptr, ctypes.byref(shape))


def topk_check(logits_ptr, stride, ctx_ptr, num_rows, width, k, out_ptr, workspace_ptr=None,
               workspace_bytes=0, row_starts_ptr=None) -> int:
    """Host-side validation only (``qsa_topk_check``); pointers are ints."""
    return lib.qsa_topk_check(logits_ptr, stride, ctx_ptr, row_starts_ptr, num_rows, width, k, out_ptr,
                              workspace_ptr, workspace_bytes)


class PreparedLogits:
    """A validated ``qsa_paged_logits`` call on fixed tensors: construction does
    every check once; each call only crosses the C ABI (for tight loops and
    benchmarks).  The tensors must stay alive and unchanged in shape."""

    def __init__(self, q, kcache, block_table, ctx_lens, row_to_req, out, *, width: int,
                 block_size: int, w=None, kscale=None, layout: int = KV_PAGED, stream=None):
        # one full checked call path on the host side, without launching
        R = int(q.shape[0])
        _require(out.dtype.is_floating_point and out.dim() == 2 and out.stride(1) == 1,
                 "out must be f32 [R, >=width]")
        self.shape = make_shape(q, kcache, block_table, width=width, block_size=block_size,
                                layout=layout, out_stride=out.stride(0) if R > 0 else width)
        self._keep = (q, kcache, block_table, ctx_lens, row_to_req, out, w, kscale)
        self._args = (_ptr(q), _ptr(w), _ptr(kcache), _ptr(kscale), _ptr(block_table),
                      _ptr(ctx_lens), _ptr(row_to_req), _ptr(out), ctypes.byref(self.shape),
                      _stream(stream))
        _raise_on(lib.qsa_paged_logits_check(*self._args[:9]))
        self.out = out

    def __call__(self, events=None):
        if events is None:
            st = lib.qsa_paged_logits(*self._args)
        else:
            st = lib.qsa_paged_logits_timed(*self._args, _event(events[0]), _event(events[1]))
        if st != OK:
            _raise_on(st)
        return self.out


class PreparedTopk:
    """A validated ``qsa_topk`` call on fixed tensors (see PreparedLogits); the
    workspace ("auto": allocated once here) is part of the prepared call."""

    def __init__(self, logits, ctx_lens, k: int, out, *, width: Optional[int] = None, row_starts=None,
                 workspace="auto", stream=None):
        R = int(logits.shape[0])
        width = int(logits.shape[1]) if width is None else int(width)
        stride = int(logits.stride(0)) if R > 0 else width
        if row_starts is not None:
            _check_rows_i32("row_starts", row_starts, R)
        ws, ws_ptr, ws_bytes = _workspace(workspace, R, width, k, logits.device, stream)
        self._keep = (logits, ctx_lens, row_starts, out, ws)
        self.workspace = ws
        self._args = (_ptr(logits), stride, _ptr(ctx_lens), _ptr(row_starts), R, width, int(k), _ptr(out), ws_ptr,
                      ws_bytes, _stream(stream))
        _raise_on(lib.qsa_topk_check(*self._args[:10]))
        self.out = out

    def __call__(self, events=None):
        if events is None:
            st = lib.qsa_topk(*self._args)
        else:
            st = lib.qsa_topk_timed(*self._args, _event(events[0]), _event(events[1]))
        if st != OK:
            _raise_on(st)
        return self.out


def paged_logits_topk_workspace_bytes(shape: LogitsShape, k: int) -> int:
    """``qsa_paged_logits_topk_workspace_bytes`` for a shape (see ``make_shape``)."""
    return int(lib.qsa_paged_logits_topk_workspace_bytes(ctypes.byref(shape), int(k)))


class PreparedLogitsTopk:
    """A validated ``qsa_paged_logits_topk`` call on fixed tensors: scoring into
    ``out`` and the top-k of those logits into ``idx``, fused where the shape
    allows; ``workspace`` "auto" allocates it once here (None: no fusion)."""

    def __init__(self, q, kcache, block_table, ctx_lens, row_to_req, out, idx, *, k: int, width: int,
                 block_size: int, w=None, kscale=None, layout: int = KV_PAGED, workspace="auto", stream=None):
        import torch
        R = int(q.shape[0])
        _require(out.dtype == torch.float32 and out.dim() == 2 and out.stride(1) == 1,
                 "out must be f32 [R, >=width]")
        _require(idx.dtype == torch.int32 and idx.is_contiguous() and tuple(idx.shape) == (R, k),
                 "idx must be contiguous int32 [R, k]")
        self.shape = make_shape(q, kcache, block_table, width=width, block_size=block_size,
                                layout=layout, out_stride=out.stride(0) if R > 0 else width)
        ws = None
        if isinstance(workspace, str):
            _require(workspace == "auto", 'workspace must be "auto", None or a device tensor')
            nbytes = paged_logits_topk_workspace_bytes(self.shape, k)
            if nbytes > 0:
                ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        elif workspace is not None:
            ws = workspace
        self.workspace = ws
        self._keep = (q, kcache, block_table, ctx_lens, row_to_req, out, idx, w, kscale, ws)
        self._args = (_ptr(q), _ptr(w), _ptr(kcache), _ptr(kscale), _ptr(block_table), _ptr(ctx_lens),
                      _ptr(row_to_req), _ptr(out), ctypes.byref(self.shape), int(k), _ptr(idx), _ptr(ws),
                      0 if ws is None else int(ws.numel()), _stream(stream))
        _raise_on(lib.qsa_paged_logits_check(*self._args[:9]))
        self.out, self.idx = out, idx

    def __call__(self, events=None):
        if events is None:
            st = lib.qsa_paged_logits_topk(*self._args)
        else:
            st = lib.qsa_paged_logits_topk_timed(*self._args, *(_event(e) for e in events))
        if st != OK:
            _raise_on(st)
        return self.out, self.idx


def paged_logits_topk(q, kcache, block_table, ctx_lens, row_to_req, *, k: int, width: int, block_size: int,
                      w=None, kscale=None, layout: int = KV_PAGED, out=None, idx=None, workspace="auto",
                      stream=None):
    """``qsa_paged_logits_topk``: (logits [R, width], indices [R, k]), exactly as
    ``paged_logits`` followed by ``topk`` on its result, fused where the shape
    allows."""
    import torch
    R = int(q.shape[0])
    if out is None:
        out = torch.empty((R, (width + 3) & ~3), dtype=torch.float32, device=q.device)[:, :width]
    if idx is None:
        idx = torch.empty((R, k), dtype=torch.int32, device=q.device)
    call = PreparedLogitsTopk(q, kcache, block_table, ctx_lens, row_to_req, out, idx, k=k, width=width,
                              block_size=block_size, w=w, kscale=kscale, layout=layout, workspace=workspace,
                              stream=stream)
    if call.workspace is not None:
        call.workspace.record_stream(_torch_stream(stream))
    return call()
