"""qsa_topk_noalloc (the library-held scratch) against qsa_topk with a caller
workspace: identical selections, on consecutive calls whose second input is
smaller, through the C ABI.  Integer index work: compared bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import qsa_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _batch(rows, W, seed, starts=False):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(0, W + 1, size=rows).astype(np.int32)
    ctx[: min(rows, 3)] = [W, 2049, 5][: min(rows, 3)]
    kinds = ["normal", "ints", "relu", "const"]
    x = np.concatenate([qsa_inputs.make_logits(1, W, [W], seed=seed + r, kind=kinds[r % 4]) for r in range(rows)])
    st = None
    if starts:
        st = (rng.integers(0, W // 4, size=rows) & ~3).astype(np.int32)
        ctx = np.minimum(ctx, W - st).astype(np.int32)
    return x, ctx, st


@pytest.mark.parametrize("first,second", [((128, 49169), (36, 30000)), ((64, 65600), (9, 9000)),
                                          ((36, 30000), (300, 9000)), ((20, 20000), (3, 5000))])
def test_noalloc_matches_workspace_call(first, second):
    import paged_mqa_logits_block_amd as m
    for i, (rows, W) in enumerate((first, second)):
        for starts in (False, True):
            x, ctx, st = _batch(rows, W, seed=17 * rows + W + i, starts=starts)
            say("noalloc", rows, W, "starts" if starts else "no starts", "call", i)
            # rows padded to a multiple of 4 floats (the ABI's stride rule)
            buf = torch.full((rows, (W + 3) & ~3), float("nan"), dtype=torch.float32, device="cuda")
            buf[:, :W] = torch.from_numpy(x).cuda()
            xt = buf[:, :W]
            ct = torch.from_numpy(ctx).cuda()
            stt = None if st is None else torch.from_numpy(st).cuda()
            out = torch.full((rows, 2048), -7, dtype=torch.int32, device="cuda")
            torch.cuda.synchronize()
            m.topk_noalloc(xt, ct, 2048, row_starts=stt, out=out)
            ref = m.topk(xt, ct, 2048, row_starts=stt, workspace="auto")
            torch.cuda.synchronize()
            assert torch.equal(out, ref), (rows, W, starts)
            o = oracle.topk(x, ctx, 2048, row_starts=st)
            g = out.cpu().numpy()
            assert np.array_equal(np.sort(g, axis=1), np.sort(o, axis=1)), (rows, W, starts)


def test_noalloc_rejects_what_qsa_topk_rejects():
    import paged_mqa_logits_block_amd as m
    xt = torch.zeros((4, 100), dtype=torch.float32, device="cuda")
    ct = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(m.QsaError) as e:
        m.topk_noalloc(xt, ct, 2049)
    assert e.value.status == m.E_UNSUPPORTED
