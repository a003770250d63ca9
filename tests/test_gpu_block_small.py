"""The single-launch path of dfs_draft_block (small, launch-bound shapes: one
workgroup per block runs the conv, head, top-K, transition scores and walk)
against the oracle on the same seeded inputs, with the end-to-end comparison
of tests/e2e_check.py (near ties scored with the oracle's scores)."""
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
    base = dict(batch=1, block=8, hidden=64, vocab=1000, top_k=8, rank=32, group=16, ksize=2, dtype="bf16")
    base.update(kw)
    return wl.Shape(**base)


def one_launch(s):
    """The library's rule for the single-launch path."""
    return (s.block <= 16 and s.top_k <= 16 and s.hidden <= 512 and s.groups * s.ksize <= 512
            and s.vocab <= 1024 and s.vocab * s.hidden <= 1 << 17 and s.block * s.vocab <= 16384 and s.rank <= 512)


SMALL_SHAPES = [
    wl.shape_of(0),                                                   # the tiny oracle-check workload, fp32
    S(),
    S(batch=3, block=16, hidden=128, vocab=1021, top_k=16, rank=64),  # longest block, K 16, ragged V
    S(batch=5, block=2, hidden=32, vocab=1024, top_k=1, rank=8),      # one draft slot, K 1, largest V
    S(batch=2, block=5, hidden=256, vocab=512, top_k=5, rank=512, group=8, ksize=4),  # four taps, largest rank
    S(batch=2, block=6, hidden=512, vocab=256, top_k=16, rank=16, group=32, ksize=1),  # conv off, largest D
    S(batch=4, block=7, hidden=96, vocab=1009, top_k=12, rank=24, dtype="f32", ksize=4, group=8),
    S(batch=2, block=16, hidden=64, vocab=17, top_k=16, rank=16),     # K close to V
]


def run(s, inp, **opts):
    dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
    dev["wg_cm"] = to_dev(wg_channel_major(inp["wg"]))
    cfg = dfs.Config.of(s)
    path = empty((s.batch, s.block), torch.int32)
    score = empty((s.batch,), torch.float32)
    ids = empty((s.rows, s.top_k), torch.int32)
    lp = empty((s.rows, s.top_k), torch.float32)
    o = {k: (to_dev(v) if isinstance(v, np.ndarray) else v) for k, v in opts.items()}
    dfs.draft_block(cfg, dev["h"], dev["anchor"], dev["wg_cm"], dev["W"], dev["P"], dev["Q"], path, score,
                    empty((dfs.workspace_size(cfg),), torch.uint8), cand_ids=ids, cand_logp=lp, **o)
    torch.cuda.synchronize()
    return [from_dev(t) for t in (path, score, ids, lp)]


@pytest.mark.parametrize("s", SMALL_SHAPES, ids=str)
def test_one_launch_block_matches_oracle(s):
    assert one_launch(s)
    inp = wl.make_inputs_for(s, 51)
    e2e.check_block_e2e(orc, s, inp, run(s, inp))


@pytest.mark.parametrize("walk", ["viterbi", "greedy", "sample"])
def test_one_launch_block_options(walk):
    """Context gate and each walk rule on the single-launch path, against the
    oracle's candidates, transitions (with the gate) and walk."""
    s = S(batch=5, block=8, hidden=128, vocab=1000, top_k=16, rank=64)
    assert one_launch(s)
    inp = wl.make_inputs_for(s, 52)
    gate = (0.5 + np.random.default_rng(53).random((s.rows, s.rank))).astype(np.float32)
    u = np.random.default_rng(54).random((s.batch, s.block)).astype(np.float32)
    extra = dict(temperature=0.8, uniforms=u) if walk == "sample" else {}
    path, score, ids, lp = run(s, inp, gate=gate, walk=walk, **extra)
    ref = orc.draft_block(s, inp["h"], inp["anchor"], inp["wg"], inp["W"], inp["P"], inp["Q"], gate=gate)
    assert np.array_equal(ids, ref["ids"])  # no near tie at rank K in these inputs
    assert np.max(np.abs(lp - ref["logp"])) <= 2e-3 * max(1.0, np.abs(ref["logp"]).max())
    for b in range(s.batch):
        rs = slice(b * s.block, (b + 1) * s.block)
        T = orc.transitions(s.with_(batch=1), int(inp["anchor"][b]), ref["ids"][rs], inp["P"], inp["Q"],
                            gate=gate[rs])
        if walk == "viterbi":
            ridx, rsc, margin = orc.viterbi(ref["logp"][rs], T)
            assert margin > 1e-3
        else:
            ridx, rsc = orc.walk(ref["logp"][rs], T, walk, 0.8, u[b].astype(np.float64) if walk == "sample" else None)
        want = [int(inp["anchor"][b])] + [int(ref["ids"][b * s.block + t, ridx[t]]) for t in range(1, s.block)]
        assert list(path[b]) == want, (walk, b)
        assert abs(score[b] - rsc) <= 2e-3 * max(1.0, abs(rsc)), (walk, b)


def test_one_launch_bad_anchor():
    s = S(batch=4)
    inp = wl.make_inputs_for(s, 55)
    inp["anchor"] = inp["anchor"].copy()
    inp["anchor"][1] = s.vocab
    inp["anchor"][2] = -3
    path, score, ids, lp = run(s, inp)
    for b in (1, 2):
        assert np.all(path[b] == -1) and np.isnan(score[b])
    ref = orc.draft_block(s.with_(batch=1), inp["h"][:s.block], inp["anchor"][:1], inp["wg"], inp["W"], inp["P"],
                          inp["Q"])
    assert list(path[0]) == list(ref["path"][0])
    assert np.array_equal(ids, orc.draft_block(s, inp["h"], np.zeros(s.batch, np.int32), inp["wg"], inp["W"],
                                               inp["P"], inp["Q"])["ids"])
