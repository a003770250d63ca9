"""dfs_draft_block_static (the allocation-free entry point) against
dfs_draft_block on a caller workspace: the same kernels, so every output is
bit-identical.  Two calls in a row share the static buffer; the second is
smaller and uses the general selector (context gate), so it reads workspace
sections the first left stale."""
import numpy as np
import pytest

import workloads as wl
from helpers import empty, from_dev, to_dev, wg_channel_major

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import block_drafter_grouped_amd as dfs  # noqa: E402


def S(**kw):
    base = dict(batch=1, block=8, hidden=256, vocab=3000, top_k=16, rank=64, group=16, ksize=2, dtype="bf16")
    base.update(kw)
    return wl.Shape(**base)


CALLS = [
    # 48 rows: the GEMM head writes its logits and segment partials into the buffer
    (S(batch=6, block=8, hidden=512, vocab=50021, top_k=16, rank=256), 41, {}),
    # then a smaller call: streaming head, gated general selector, greedy walk
    (S(batch=1, block=8, hidden=256, vocab=20011, top_k=12, rank=64), 42, {"gate": True, "walk": "greedy"}),
]


def run(s, seed, opts, static):
    inp = wl.make_inputs_for(s, seed)
    dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
    wg = to_dev(wg_channel_major(inp["wg"]))
    cfg = dfs.Config.of(s)
    assert dfs.workspace_size(cfg) <= dfs.STATIC_WORKSPACE_BYTES
    kw = {}
    if opts.get("gate"):
        g = np.random.default_rng(seed).random((s.rows, s.rank)).astype(np.float32) + 0.5
        kw["gate"] = to_dev(g)
    if "walk" in opts:
        kw["walk"] = opts["walk"]
    path = empty((s.batch, s.block), torch.int32)
    score = empty((s.batch,), torch.float32)
    ids = empty((s.rows, s.top_k), torch.int32)
    lp = empty((s.rows, s.top_k), torch.float32)
    if static:
        dfs.draft_block_static(cfg, dev["h"], dev["anchor"], wg, dev["W"], dev["P"], dev["Q"], path, score,
                               cand_ids=ids, cand_logp=lp, **kw)
    else:
        ws = empty((dfs.workspace_size(cfg),), torch.uint8)
        dfs.draft_block(cfg, dev["h"], dev["anchor"], wg, dev["W"], dev["P"], dev["Q"], path, score, ws,
                        cand_ids=ids, cand_logp=lp, **kw)
    torch.cuda.synchronize()
    return [from_dev(t) for t in (path, score, ids, lp)]


def test_static_workspace_matches_caller_workspace():
    got = [run(s, seed, opts, static=True) for s, seed, opts in CALLS]  # two calls in a row
    for (s, seed, opts), g in zip(CALLS, got):
        want = run(s, seed, opts, static=False)
        for a, b in zip(g, want):
            assert np.array_equal(a, b, equal_nan=True), str(s)
    # and once more, the large call after the small one
    s, seed, opts = CALLS[0]
    again = run(s, seed, opts, static=True)
    for a, b in zip(again, got[0]):
        assert np.array_equal(a, b, equal_nan=True)
