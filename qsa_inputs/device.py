"""Copy a ``PagedInputs`` batch to device tensors (bytes unchanged)."""
from __future__ import annotations

import types

import numpy as np


def to_device(inp, device="cuda"):
    import torch

    def t(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)

    if inp.dtype in ("bf16", "fp16"):
        td = torch.bfloat16 if inp.dtype == "bf16" else torch.float16
        q = t(inp.q.view(np.int16)).view(td)
        kc = t(inp.kcache.view(np.int16)).view(td)
    else:
        q = t(inp.q).view(torch.float8_e4m3fn)
        kc = t(inp.kcache) if inp.layout != "paged" else t(inp.kcache).view(torch.float8_e4m3fn)
    return types.SimpleNamespace(
        q=q, w=t(inp.w), kcache=kc, kscale=t(inp.kscale), block_table=t(inp.block_table),
        ctx_lens=t(inp.ctx_lens.astype(np.int32)), row_to_req=t(inp.row_to_req),
        width=inp.width, block_size=inp.block_size, topk=inp.topk,
        layout={"paged": 0, "copacked": 1, "copacked_shuffled": 2}[inp.layout])
