"""Seeded synthetic inputs for paged MQA-logits scoring and per-row top-k.

This module only *draws* inputs: it holds none of the scoring or selection
arithmetic.  Both the CPU oracle and the HIP path are fed from here, so every
comparison between them is made on identical bytes.

Workload shapes follow the pages:

* "Tiny" / "Decode verify": MTP-3 verification gives every request 4 query rows
  that share the request's keys (ROCm/ATOM PR #2651, Motivation and Changes).
* "Single-row decode, mixed lengths": one row per request, 4 index heads
  zero-padded to the MFMA width of 16 (sglang PR #48649, Modifications), table
  width 65,600 compressed columns (vLLM PR #62589, Overview).
* "FP8 paged": e4m3 queries and keys with a per-key f32 scale, f32 head
  weights, block-flat co-packed blocks of 64 keys then 64 scales
  (ROCm/aiter PR #4221, commit "extend fp8_paged_mqa_logits ... KVBlockSize>=1",
  and Motivation).
* "Prefill chunk": a 16K-row chunk at positions 98,304.. of one request
  (vLLM PR #62589, MI355X comment table "16K chunk at 96K"; ATOM PR #2651,
  Performance "prefill[bs=1 tok=16384 ctx=98304]").

Layouts handed to both sides:

* q       : bf16 bits ``uint16 [R, H, D]`` or e4m3fn codes ``uint8 [R, H, D]``
* w       : ``float32 [R, H]`` or ``None`` (meaning every weight is 1)
* kcache  : paged bf16 ``uint16 [NB, B, D]``; paged fp8 ``uint8 [NB, B, D]``
            with ``kscale float32 [NB, B]``; co-packed fp8 ``uint8 [NB, B*(D+4)]``
            (B*D key bytes, key c at byte c*D, then B little-endian f32 scales)
* block_table : ``int32 [num_reqs, max_blocks]``
* ctx_lens    : ``int32 [R]`` visible columns per row
* row_to_req  : ``int32 [R]``
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

HEAD_DIM = 128

BF16_NAN = np.uint16(0x7FC0)
FP16_NAN = np.uint16(0x7E00)
FP8_NAN = np.uint8(0x7F)

CONFIG_NAMES = ("tiny", "decode_verify", "single_row_mixed", "fp8_paged", "prefill_chunk")
# the same shapes with fp16 q and keys (the pages' fp16 callers)
FP16_CONFIG_NAMES = ("decode_verify_fp16", "prefill_chunk_fp16")
# fp8_paged with one key per table entry (the per-token co-packed layout)
KVB1_CONFIG_NAMES = ("fp8_paged_kvb1",)
# fp8_paged with the keys of every co-packed block preshuffled in 16x16-byte tiles
SHUFFLED_CONFIG_NAMES = ("fp8_paged_shuffled",)
# decode_verify with head dim 64
D64_CONFIG_NAMES = ("decode_verify_d64",)
# fp8_paged with a ragged number of verify rows per request (1..8, mean 4.5)
RAGGED_CONFIG_NAMES = ("fp8_paged_ragged",)


@dataclasses.dataclass
class PagedInputs:
    """One batch of paged-logits inputs plus the top-k size."""

    name: str
    dtype: str  # "bf16", "fp16" or "fp8"
    layout: str  # "paged", "copacked" or "copacked_shuffled"
    num_heads: int
    head_dim: int
    block_size: int
    max_blocks: int
    width: int
    topk: int
    q: np.ndarray
    w: Optional[np.ndarray]
    kcache: np.ndarray
    kscale: Optional[np.ndarray]
    block_table: np.ndarray
    ctx_lens: np.ndarray
    row_to_req: np.ndarray
    kv_lens: np.ndarray  # per request: columns that hold keys

    @property
    def num_rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_reqs(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.kcache.shape[0])

    def ctx_eff(self) -> np.ndarray:
        """Visible columns per row after clamping to the table and the width."""
        cap = min(self.width, self.max_blocks * self.block_size)
        return np.clip(self.ctx_lens.astype(np.int64), 0, cap)

    def key_bytes_per_col(self) -> int:
        if self.dtype in ("bf16", "fp16"):
            return 2 * self.head_dim
        return self.head_dim + (4 if (self.layout != "paged" or self.kscale is not None) else 0)


# ----------------------------------------------------------------------------
# element encoders (input synthesis only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest IEEE binary16 (numpy's cast, ties to even);
    returns the bits."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16).copy()


def f32_to_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """Saturate to +-448 and round to the nearest OCP e4m3fn code (ties to even).

    Uses torch's float8_e4m3fn cast, a library routine, for the rounding.
    """
    import torch

    t = torch.from_numpy(np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def shuffle_keys_16x16(k8: np.ndarray) -> np.ndarray:
    """Block-flat fp8 keys [blocks, B, D] -> the preshuffled key section
    [blocks, B*D]: each group of 16 slots becomes D/16 chunks of 16 slots x 16
    bytes (a layout transform of the input bytes only)."""
    nb, B, D = k8.shape
    assert B % 16 == 0 and D % 16 == 0
    g = k8.reshape(nb, B // 16, 16, D // 16, 16)          # block, group, slot, chunk, byte
    return np.ascontiguousarray(g.transpose(0, 1, 3, 2, 4)).reshape(nb, B * D)


# ----------------------------------------------------------------------------
# generic builder
# ----------------------------------------------------------------------------

def build(
    *,
    name: str,
    seed: int,
    req_rows: Sequence[int],
    ctx_rows: Sequence[int],
    kv_lens: Optional[Sequence[int]] = None,
    num_heads: int = 4,
    real_heads: Optional[int] = None,
    block_size: int = 16,
    dtype: str = "bf16",
    layout: str = "paged",
    weights: bool = False,
    fp8_scale: bool = True,
    max_blocks: Optional[int] = None,
    width: Optional[int] = None,
    pool: Optional[int] = None,
    topk: int = 2048,
    poison: bool = False,
    shuffle_rows: bool = False,
    head_dim: int = HEAD_DIM,
) -> PagedInputs:
    """Draw one batch.

    ``req_rows[i]`` rows belong to request i (request-major unless
    ``shuffle_rows``).  ``ctx_rows`` gives each row's visible column count (in
    the final row order).  ``kv_lens[i]`` is how many key columns request i holds
    (default: the max ctx of its rows).  Heads ``>= real_heads`` of q are zero.

    With ``poison`` the unused table slots point at an extra block filled with
    NaN, and key slots of a request's last block past ``kv_lens`` hold NaN, so a
    kernel that reads keys it must not touch produces NaN where it is compared.
    """
    rng = np.random.default_rng(seed)
    req_rows = [int(n) for n in req_rows]
    num_reqs = len(req_rows)
    R = int(sum(req_rows))
    row_to_req = np.repeat(np.arange(num_reqs, dtype=np.int32), req_rows)
    if shuffle_rows:
        row_to_req = row_to_req[rng.permutation(R)].astype(np.int32)
    ctx = np.asarray(ctx_rows, dtype=np.int32).reshape(R)
    if kv_lens is None:
        kv = np.zeros(num_reqs, dtype=np.int64)
        for r in range(R):
            kv[row_to_req[r]] = max(kv[row_to_req[r]], int(ctx[r]))
    else:
        kv = np.asarray(kv_lens, dtype=np.int64).reshape(num_reqs)
    B = int(block_size)
    blocks_per_req = [(int(n) + B - 1) // B for n in kv]
    if max_blocks is None:
        max_blocks = max(1, max(blocks_per_req))
    if width is None:
        width = max_blocks * B
    needed = int(sum(blocks_per_req))
    if pool is None:
        pool = max(needed, 1)
    assert pool >= needed, (pool, needed)
    num_blocks = pool + (1 if poison else 0)
    H = int(num_heads)
    D = int(head_dim)
    if real_heads is None:
        real_heads = H

    # block table: a seeded permutation of the pool, handed out in request order
    perm = rng.permutation(pool).astype(np.int32)
    fill = pool if poison else 0
    bt = np.full((num_reqs, max_blocks), fill, dtype=np.int32)
    pos = 0
    for i, nb in enumerate(blocks_per_req):
        assert nb <= max_blocks
        bt[i, :nb] = perm[pos:pos + nb]
        pos += nb

    # queries
    qf = rng.standard_normal((R, H, D), dtype=np.float32)
    qf[:, real_heads:, :] = 0.0
    if dtype == "bf16":
        q = f32_to_bf16_bits(qf)
    elif dtype == "fp16":
        q = f32_to_fp16_bits(qf)
    elif dtype == "fp8":
        q = f32_to_e4m3fn_codes(qf)
    else:
        raise ValueError(dtype)

    w = rng.uniform(0.0, 1.0, size=(R, H)).astype(np.float32) if weights else None

    # keys
    kf = rng.standard_normal((num_blocks, B, D), dtype=np.float32)
    kscale = None
    if dtype in ("bf16", "fp16"):
        assert layout == "paged"
        kc = f32_to_bf16_bits(kf) if dtype == "bf16" else f32_to_fp16_bits(kf)
        nan = BF16_NAN if dtype == "bf16" else FP16_NAN
        if poison:
            kc[pool] = nan
            for i, n in enumerate(kv):
                if n % B and blocks_per_req[i]:
                    kc[bt[i, blocks_per_req[i] - 1], n % B:, :] = nan
    else:
        if fp8_scale:
            amax = np.max(np.abs(kf), axis=2)
            s = (amax / np.float32(448.0)).astype(np.float32)
            s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        else:
            s = np.ones((num_blocks, B), dtype=np.float32)
        k8 = f32_to_e4m3fn_codes(kf / s[:, :, None])
        if poison:
            k8[pool] = FP8_NAN
            s[pool] = np.float32(np.nan)
            for i, n in enumerate(kv):
                if n % B and blocks_per_req[i]:
                    blk = bt[i, blocks_per_req[i] - 1]
                    k8[blk, n % B:, :] = FP8_NAN
                    s[blk, n % B:] = np.float32(np.nan)
        if layout == "paged":
            kc = k8
            kscale = s
        elif layout in ("copacked", "copacked_shuffled"):
            kc = np.empty((num_blocks, B * (D + 4)), dtype=np.uint8)
            if layout == "copacked":
                kc[:, : B * D] = k8.reshape(num_blocks, B * D)
            else:
                kc[:, : B * D] = shuffle_keys_16x16(k8)
            kc[:, B * D:] = s.astype("<f4").view(np.uint8).reshape(num_blocks, 4 * B)
        else:
            raise ValueError(layout)

    return PagedInputs(
        name=name, dtype=dtype, layout=layout, num_heads=H, head_dim=D,
        block_size=B, max_blocks=int(max_blocks), width=int(width), topk=int(topk),
        q=q, w=w, kcache=kc, kscale=kscale, block_table=bt, ctx_lens=ctx,
        row_to_req=row_to_req.astype(np.int32), kv_lens=kv.astype(np.int64),
    )


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

def make_config(name: str, seed: Optional[int] = None, poison: bool = False) -> PagedInputs:
    """The five named workloads, seeded 1..5 by default; fp16 variants of
    decode_verify and prefill_chunk (same shapes and recipe, seeds 6 and 7);
    fp8_paged with one key per block (seed 8); fp8_paged with preshuffled keys
    (seed 9); decode_verify with head dim 64 (seed 10); fp8_paged with 1..8 verify
    rows per request (seed 11)."""
    if name == "fp8_paged_kvb1":
        kv_len, next_n, reqs = 32768, 4, 16
        ctx = [kv_len - next_n + n + 1 for _ in range(reqs) for n in range(next_n)]
        return build(name=name, seed=8 if seed is None else seed, req_rows=[next_n] * reqs,
                     ctx_rows=ctx, kv_lens=[kv_len] * reqs, num_heads=64, block_size=1,
                     dtype="fp8", layout="copacked", weights=True, max_blocks=kv_len,
                     width=32768, topk=2048, poison=poison)
    if name == "fp8_paged_shuffled":
        kv_len, next_n, reqs = 32768, 4, 16
        ctx = [kv_len - next_n + n + 1 for _ in range(reqs) for n in range(next_n)]
        return build(name=name, seed=9 if seed is None else seed, req_rows=[next_n] * reqs,
                     ctx_rows=ctx, kv_lens=[kv_len] * reqs, num_heads=64, block_size=64,
                     dtype="fp8", layout="copacked_shuffled", weights=True, max_blocks=512,
                     width=32768, topk=2048, poison=poison)
    if name == "fp8_paged_ragged":
        # confidence-trimmed MTP verify: next_n drawn per request from 1..8
        # (mean 4.5); row n of a request sees kv_len - next_n + n + 1 columns
        rng = np.random.default_rng(11 if seed is None else seed)
        kv_len, reqs = 32768, 16
        next_n = rng.integers(1, 9, size=reqs)
        ctx = [kv_len - int(nn) + n + 1 for nn in next_n for n in range(int(nn))]
        return build(name=name, seed=int(rng.integers(1 << 31)), req_rows=[int(x) for x in next_n],
                     ctx_rows=ctx, kv_lens=[kv_len] * reqs, num_heads=64, block_size=64,
                     dtype="fp8", layout="copacked", weights=True, max_blocks=512,
                     width=32768, topk=2048, poison=poison)
    if name == "decode_verify_d64":
        rng = np.random.default_rng(10 if seed is None else seed)
        ctx_req = rng.integers(16000, 32000, size=9, endpoint=True)
        return build(name=name, seed=int(rng.integers(1 << 31)), req_rows=[4] * 9,
                     ctx_rows=np.repeat(ctx_req, 4), num_heads=4, head_dim=64, block_size=16,
                     topk=2048, poison=poison)
    if name in FP16_CONFIG_NAMES:
        base = name[: -len("_fp16")]
        return make_config_dtype(base, "fp16", seed=(6 if base == "decode_verify" else 7) if seed is None else seed,
                                 poison=poison)
    return make_config_dtype(name, "bf16", seed=seed, poison=poison)


def make_config_dtype(name: str, dtype: str, seed: Optional[int] = None, poison: bool = False) -> PagedInputs:
    """One named workload; ``dtype`` applies to the bf16 ones (bf16 or fp16)."""
    if name == "tiny":
        # 2 requests x 4 rows, contexts 1000 and 3000, block 16, pool of 256 blocks
        return build(name=name, seed=1 if seed is None else seed, req_rows=[4, 4],
                     ctx_rows=[1000] * 4 + [3000] * 4, num_heads=4, block_size=16,
                     pool=256, topk=256, poison=poison)
    if name == "decode_verify":
        rng = np.random.default_rng(2 if seed is None else seed)
        ctx_req = rng.integers(16000, 32000, size=9, endpoint=True)
        return build(name=name, seed=int(rng.integers(1 << 31)), req_rows=[4] * 9,
                     ctx_rows=np.repeat(ctx_req, 4), num_heads=4, block_size=16,
                     topk=2048, dtype=dtype, poison=poison)
    if name == "single_row_mixed":
        rng = np.random.default_rng(3 if seed is None else seed)
        ctx_req = np.floor(np.exp(rng.uniform(math.log(5000), math.log(65600), size=64)))
        ctx_req = np.minimum(ctx_req, 65600).astype(np.int64)
        return build(name=name, seed=int(rng.integers(1 << 31)), req_rows=[1] * 64,
                     ctx_rows=ctx_req, num_heads=16, real_heads=4, block_size=64,
                     max_blocks=1025, width=65600, topk=2048, poison=poison)
    if name == "fp8_paged":
        # next_n = 4 MTP rows per request; row n sees kv_len - next_n + n + 1 columns
        kv_len, next_n, reqs = 32768, 4, 16
        ctx = [kv_len - next_n + n + 1 for _ in range(reqs) for n in range(next_n)]
        return build(name=name, seed=4 if seed is None else seed, req_rows=[next_n] * reqs,
                     ctx_rows=ctx, kv_lens=[kv_len] * reqs, num_heads=64, block_size=64,
                     dtype="fp8", layout="copacked", weights=True, max_blocks=512,
                     width=32768, topk=2048, poison=poison)
    if name == "prefill_chunk":
        pos = np.arange(98304, 98304 + 16384, dtype=np.int64)
        ctx = (pos + 1) // 4
        return build(name=name, seed=5 if seed is None else seed, req_rows=[16384],
                     ctx_rows=ctx, kv_lens=[28672], num_heads=4, block_size=64,
                     max_blocks=448, width=28672, topk=2048, dtype=dtype, poison=poison)
    raise KeyError(name)


# ----------------------------------------------------------------------------
# synthetic logits for selection-only tests
# ----------------------------------------------------------------------------

def make_logits(rows: int, width: int, ctx: Sequence[int], seed: int, kind: str = "normal",
                tail: str = "neginf") -> np.ndarray:
    """A float32 ``[rows, width]`` logits buffer.

    ``kind``: "normal" (distinct with high probability), "ints" (small integers,
    many exact ties), "const" (every visible value equal), "zeros" (a mix of
    +0.0 and -0.0), "relu" (many exact zeros, like summed ReLU outputs),
    "offset" (values in [30000, 30000.49] plus seven distinct larger ones per
    row, 30000.5 + 0.01 i: a range about 50,000 times narrower than its
    largest value), "tiny" (normal floats within 4,096 ulp of 1e-36: a range
    below 1e-39, too narrow for 2,048 buckets of float32 width).
    ``tail`` fills ``[ctx, width)``: "neginf" or "nan".
    """
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.standard_normal((rows, width), dtype=np.float32) * np.float32(10.0)
    elif kind == "ints":
        x = rng.integers(-8, 8, size=(rows, width)).astype(np.float32)
    elif kind == "const":
        x = np.full((rows, width), 3.25, dtype=np.float32)
    elif kind == "zeros":
        x = np.where(rng.integers(0, 2, size=(rows, width)) == 1, np.float32(-0.0), np.float32(0.0))
        x = x.astype(np.float32)
        x[:, ::7] = np.float32(1.5)
    elif kind == "relu":
        x = np.maximum(rng.standard_normal((rows, width), dtype=np.float32), np.float32(0.0))
    elif kind == "offset":
        x = (np.float32(30000.0) + np.float32(0.49) * rng.random((rows, width), dtype=np.float32)).astype(np.float32)
        for r, c in enumerate(np.asarray(ctx, dtype=np.int64).reshape(rows)):
            c = int(min(max(c, 0), width))
            cols = rng.permutation(c)[:7]
            x[r, cols] = (np.float32(30000.5) + np.float32(0.01) * np.arange(len(cols), dtype=np.float32)).astype(np.float32)
    elif kind == "tiny":
        base = np.array([1e-36], dtype=np.float32).view(np.uint32)[0]
        x = (base + rng.integers(0, 4096, size=(rows, width)).astype(np.uint32)).view(np.float32)
    else:
        raise ValueError(kind)
    fillv = np.float32(-np.inf) if tail == "neginf" else np.float32(np.nan)
    ctx = np.asarray(ctx, dtype=np.int64).reshape(rows)
    for r in range(rows):
        c = int(min(max(ctx[r], 0), width))
        x[r, c:] = fillv
    return x
