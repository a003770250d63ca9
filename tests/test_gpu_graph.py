"""A whole draft block captured in a HIP graph (through torch.cuda.graph) and
replayed: every replay must reproduce the eager result bit for bit, and the
replays of the default selector are also compared with the oracle on the
same seeded inputs.  The
library allocates, frees and synchronises nothing and takes the caller's
stream, so a caller can capture a step to cut launch overhead on
launch-bound shapes.  Between replays the test runs its own eager work
(clobbering the outputs) and synchronises."""
import numpy as np
import pytest

import workloads as wl
from helpers import empty, from_dev, to_dev, wg_channel_major

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import block_drafter_grouped_amd as dfs  # noqa: E402
import e2e_check as e2e  # noqa: E402
import oracle as orc  # noqa: E402


def S(**kw):
    base = dict(batch=1, block=8, hidden=256, vocab=3000, top_k=16, rank=64, group=16, ksize=2, dtype="bf16")
    base.update(kw)
    return wl.Shape(**base)


@pytest.mark.parametrize("s", [
    S(batch=1, block=8, hidden=512, vocab=20000, top_k=16, rank=256),   # streaming head, fused selector
    S(batch=6, block=8, hidden=256, vocab=9001, top_k=16, rank=64),     # GEMM head (512-wide tiles), segment merge
    S(batch=20, block=8, hidden=256, vocab=9001, top_k=16, rank=64),    # GEMM head (256 x 256 tiles), segment merge
    S(batch=2, block=6, hidden=128, vocab=3000, top_k=24, rank=32),     # K > 16: slice top-K, general selector
    wl.shape_of(0),                                                    # fp32
], ids=str)
def test_draft_block_graph_replay(s):
    replay_and_check(s, {})


@pytest.mark.parametrize("s,walk", [
    (S(batch=1, block=8, hidden=512, vocab=20000, top_k=16, rank=256), "greedy"),   # fused selector, gated
    (S(batch=3, block=8, hidden=256, vocab=7001, top_k=16, rank=64), "sample"),     # GEMM head, fused selector
    (S(batch=2, block=20, hidden=128, vocab=3000, top_k=24, rank=32), "viterbi"),   # general selector, gated
], ids=str)
def test_draft_block_graph_replay_with_options(s, walk):
    """The same with a context gate and each walk rule: every replay gives
    the eager result bit for bit (the oracle comparison of these options is
    the parity suite's)."""
    rng = np.random.default_rng(29)
    opts = dict(gate=to_dev((0.5 + rng.random((s.rows, s.rank))).astype(np.float32)), walk=walk)
    if walk == "sample":
        opts.update(temperature=0.8, uniforms=to_dev(rng.random((s.batch, s.block)).astype(np.float32)))
    replay_and_check(s, opts)


def replay_and_check(s, opts):
    inp = wl.make_inputs_for(s, 23)
    dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
    dev["wg_cm"] = to_dev(wg_channel_major(inp["wg"]))
    cfg = dfs.Config.of(s)
    ws = empty((dfs.workspace_size(cfg),), torch.uint8)
    path = empty((s.batch, s.block), torch.int32)
    score = empty((s.batch,), torch.float32)
    ids = empty((s.rows, s.top_k), torch.int32)
    lp = empty((s.rows, s.top_k), torch.float32)

    def step():
        dfs.draft_block(cfg, dev["h"], dev["anchor"], dev["wg_cm"], dev["W"], dev["P"], dev["Q"], path, score, ws,
                        cand_ids=ids, cand_logp=lp, **opts)

    step()
    torch.cuda.synchronize()
    want = [from_dev(t).copy() for t in (path, score, ids, lp)]

    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        step()  # once eagerly on the capture stream
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (path, ids):
            t.fill_(-7)
        for t in (score, lp):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [from_dev(t) for t in (path, score, ids, lp)]
        if not opts:
            e2e.check_block_e2e(orc, s, inp, got)
        for a, b in zip(got, want):
            assert np.array_equal(a, b, equal_nan=True), f"replay {rep}"
