"""GPU parity of every libdflash2 entry point against the fp64 oracle.

FED mode feeds both sides the same intermediate (the bit-exact gates):
top-K ids of the GPU's own fp32 logits vs a full sort, the walk on the GPU's
candidates vs the oracle walk, scores to 1e-4.  E2E mode runs the whole block
on both sides from the same seeded inputs: conv, logits and lse to a relative
2e-3, ids and paths equal unless a near tie explains the difference.
"""
import math

import numpy as np
import pytest

import workloads as wl
from helpers import as_f64, empty, from_dev, ids_match_or_explained, rel_err, to_dev, topk_of, wg_channel_major

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import block_drafter_grouped_amd as dfs  # noqa: E402
import e2e_check as e2e  # noqa: E402
import oracle as orc  # noqa: E402

TOL = 2e-3         # relative (conv, logits, lse), the stated tolerance
SCORE_TOL = 1e-4   # absolute, path scores in FED mode
NEAR_TIE = 1e-4    # path margin below which two paths count as tied


def S(**kw):
    base = dict(batch=1, block=8, hidden=256, vocab=3000, top_k=16, rank=64, group=16, ksize=2, dtype="bf16")
    base.update(kw)
    return wl.Shape(**base)


def wsbuf(cfg):
    n = dfs.workspace_size(cfg)
    assert n > 0
    return empty((n,), torch.uint8)


_CACHE = {}


def cfg_inputs(cfg_id):
    if cfg_id not in _CACHE:
        _CACHE.clear()  # keep one full-size workload resident at a time
        inp = wl.make_inputs(cfg_id)
        dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
        dev["wg_cm"] = to_dev(wg_channel_major(inp["wg"]))
        _CACHE[cfg_id] = (inp, dev)
    return _CACHE[cfg_id]


def tdtype(s):
    return torch.int16 if s.dtype == "bf16" else torch.float32


# ============================================================== conv

CONV_SHAPES = [
    wl.WORKLOADS[0],
    wl.WORKLOADS[0].with_(dtype="bf16"),
    S(batch=3, block=5, hidden=96, group=8, ksize=4),
    S(batch=2, block=7, hidden=256, group=32, ksize=1),
    S(batch=13, block=8, hidden=512),
    S(batch=2, block=6, hidden=128, ksize=4, dtype="f32"),
    S(batch=3, block=16, hidden=64, group=64, ksize=2),
    S(batch=2, block=5, hidden=96, ksize=1, dtype="f32"),
    S(batch=2, block=8, hidden=8192),  # the largest bf16 hidden size
    # one-launch conv at up to 8 rows: two load passes (D 8192), more causal
    # taps than threads (groups of 64), one tap with the fp32 output (the
    # second tap slot weighted 0), a 3-row block
    S(batch=1, block=8, hidden=8192),
    S(batch=1, block=8, hidden=512, group=64),
    S(batch=1, block=6, hidden=3072, ksize=1),
    S(batch=1, block=3, hidden=2048, group=32),
    # split-D conv (more than 16 rows): groups of 4 channels (the per-channel
    # apply), four taps
    S(batch=3, block=8, hidden=128, group=4),
    S(batch=5, block=8, hidden=256, ksize=4),
]


@pytest.mark.parametrize("s", CONV_SHAPES + [1, 3], ids=str)
def test_conv_parity(s):
    if isinstance(s, int):
        inp = wl.make_inputs(s, parts=("h", "wg"))
        s = wl.shape_of(s)
    else:
        inp = wl.make_inputs_for(s, 5, parts=("h", "wg"))
    cfg = dfs.Config.of(s)
    h = to_dev(inp["h"])
    wg = to_dev(wg_channel_major(inp["wg"]))
    y = empty((s.rows, s.hidden), tdtype(s))
    yf = empty((s.rows, s.hidden), torch.float32)
    ws = wsbuf(cfg)
    dfs.conv(cfg, h, wg, y, ws, y_f32=yf)
    torch.cuda.synchronize()
    _, _, yhat = orc.conv(s, inp["h"], inp["wg"])
    yf_h = from_dev(yf)
    assert rel_err(yf_h, yhat) <= TOL
    y_h = from_dev(y)
    if s.dtype == "bf16":
        assert np.array_equal(y_h, wl.bf16_bits(yf_h))
    else:
        assert np.array_equal(y_h, yf_h)
    # the parity output does not change the product output
    y2 = empty((s.rows, s.hidden), tdtype(s))
    dfs.conv(cfg, h, wg, y2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(y2), y_h)


@pytest.mark.parametrize("s", [
    S(batch=1, block=8, hidden=256),                       # <= 16 rows
    S(batch=5, block=8, hidden=128, group=8, ksize=4),     # > 16 rows
    S(batch=2, block=8, hidden=128, ksize=1),              # one tap
    S(batch=2, block=6, hidden=96, ksize=2, dtype="f32"),
], ids=str)
def test_conv_layers_parity(s):
    """dfs_conv_layers: each layer equals dfs_conv on that layer alone (same
    kernels, bit for bit), whose fp32 result matches the oracle conv of that
    layer."""
    L = 3
    layers = [wl.make_inputs_for(s, 200 + l, parts=("h", "wg")) for l in range(L)]
    cfg = dfs.Config.of(s)
    h = to_dev(np.stack([x["h"] for x in layers]))
    wg = to_dev(np.stack([wg_channel_major(x["wg"]) for x in layers]))
    y = empty((L, s.rows, s.hidden), tdtype(s))
    ws = empty((dfs.conv_layers_workspace_size(cfg, L),), torch.uint8)
    dfs.conv_layers(cfg, L, h, wg, y, ws)
    torch.cuda.synchronize()
    got = from_dev(y)
    for l, x in enumerate(layers):
        y1 = empty((s.rows, s.hidden), tdtype(s))
        yf1 = empty((s.rows, s.hidden), torch.float32)
        dfs.conv(cfg, to_dev(x["h"]), to_dev(wg_channel_major(x["wg"])), y1, wsbuf(cfg), y_f32=yf1)
        torch.cuda.synchronize()
        assert np.array_equal(got[l], from_dev(y1)), l
        # the fp32 result before rounding against the exact conv of the layer
        _, _, yhat = orc.conv(s, x["h"], x["wg"])
        assert rel_err(from_dev(yf1), yhat) <= TOL, l


# ============================================================== head + top-K (FED)

HEAD_SHAPES = [
    wl.WORKLOADS[0],
    S(block=8, hidden=64, vocab=1000, top_k=4),
    S(block=3, hidden=128, vocab=4097, top_k=16),
    S(batch=5, block=4, hidden=256, vocab=20000, top_k=16),
    S(block=8, hidden=512, vocab=5000, top_k=1),
    S(block=8, hidden=256, vocab=3000, top_k=17),
    S(block=8, hidden=256, vocab=3000, top_k=64),
    S(batch=5, block=1 + 1, hidden=64, vocab=16, top_k=16),
    S(block=6, hidden=96, vocab=3001, top_k=7, dtype="f32"),
    # more than 8 rows: the GEMM head and the slice top-K of its logits
    S(batch=3, block=3, hidden=32, vocab=100, top_k=16),
    S(batch=4, block=8, hidden=96, vocab=3001, top_k=16),
    S(batch=20, block=8, hidden=128, vocab=70000, top_k=64),
    S(batch=40, block=8, hidden=64, vocab=5000, top_k=5),
    S(batch=10, block=10, hidden=128, vocab=3001, top_k=16),  # 100 rows: a partial 128-row pass
    S(batch=32, block=8, hidden=64, vocab=3001, top_k=16),    # one whole 256-row pass
    S(batch=32, block=8, hidden=32, vocab=2000, top_k=8),     # 32-channel stages, whole 256-row pass
    S(batch=20, block=8, hidden=96, vocab=9001, top_k=16),    # 32-channel stages, partial 256-row pass
    S(batch=40, block=8, hidden=128, vocab=70001, top_k=16),  # two row passes, segment merge
]


def run_head(s, y_np, W_np, W_dev=None, with_logits=True):
    cfg = dfs.Config.of(s)
    y = to_dev(y_np)
    W = W_dev if W_dev is not None else to_dev(W_np)
    ids = empty((s.rows, s.top_k), torch.int32)
    lp = empty((s.rows, s.top_k), torch.float32)
    lse = empty((s.rows,), torch.float32)
    logits = empty((s.rows, s.vocab), torch.float32) if with_logits else None
    dfs.head_topk(cfg, y, W, ids, lp, lse, wsbuf(cfg), logits_f32=logits)
    torch.cuda.synchronize()
    return (from_dev(ids), from_dev(lp), from_dev(lse), from_dev(logits) if with_logits else None)


def check_head_fed(s, y_np, W_np, W_dev=None, rows=None):
    ids, lp, lse, logits = run_head(s, y_np, W_np, W_dev)
    # (i) ids are exactly the top-K of the GPU's own fp32 logits, by a direct sort
    rid, rlse = topk_of(logits, s.top_k)
    assert np.array_equal(ids, rid)
    assert rel_err(lse, rlse) <= 1e-5
    # scores are logit - lse in fp32
    want = (np.take_along_axis(logits, ids, 1) - lse[:, None]).astype(np.float32)
    assert np.array_equal(lp, want)
    # (ii) logits, lse and ids against the oracle head fed the same y: every
    # row, or the sampled rows one by one
    if rows is None:
        ref = orc.head(s, y_np, W_np, want_logits=True)
        assert rel_err(logits, ref["logits"]) <= TOL
        assert rel_err(lse, ref["lse"]) <= TOL
        assert not ids_match_or_explained(ids, ref["ids"], lambda i: ref["logits"][i], tol_abs=TOL * 3.0)
    else:
        for r in rows:
            ref = orc.head(s, y_np, W_np, r0=r, nr=1, want_logits=True)
            assert rel_err(logits[r], ref["logits"][0]) <= TOL
            assert rel_err(lse[r], ref["lse"][0]) <= TOL
            assert not ids_match_or_explained(ids[r:r + 1], ref["ids"], lambda i: ref["logits"][0],
                                              tol_abs=TOL * 3.0)
    check_timed_mode(s, y_np, W_np, W_dev, ids, lp, lse, logits)


def check_timed_mode(s, y_np, W_np, W_dev, ids, lp, lse, logits):
    """The timed mode (no logits written) returns the same candidates, score
    and lse bits as the parity mode: both run the same kernels, only the
    logits go to the workspace instead of the caller's buffer."""
    ids2, lp2, lse2, _ = run_head(s, y_np, W_np, W_dev, with_logits=False)
    assert np.array_equal(ids2, ids) and np.array_equal(lp2, lp) and np.array_equal(lse2, lse)


@pytest.mark.parametrize("s", HEAD_SHAPES, ids=str)
def test_head_topk_fed(s):
    inp = wl.make_inputs_for(s, 11, parts=("h", "W"))
    check_head_fed(s, inp["h"], inp["W"])


# The limits of the configuration: the largest vocabulary (2^21, K 64: the
# K > 16 merge over 256 chunk lists) and the largest bf16 hidden size (8192:
# the streaming head keeps 128 KB of hidden rows in LDS; the GEMM head runs
# 128 stages per tile).  Checked against the oracle on sampled rows.
MAX_HEAD_SHAPES = [
    S(block=4, hidden=64, vocab=1 << 21, top_k=64),
    # the GEMM head's segment merge at the largest vocabulary: 32 tiles per
    # list, 16 384 segments per row
    S(batch=3, block=8, hidden=64, vocab=1 << 21, top_k=16),
    S(block=8, hidden=8192, vocab=20000, top_k=16),
    S(batch=3, block=8, hidden=8192, vocab=20000, top_k=16),
]


@pytest.mark.parametrize("s", MAX_HEAD_SHAPES, ids=str)
def test_head_topk_fed_max_sizes(s):
    inp = wl.make_inputs_for(s, 17, parts=("h", "W"))
    check_head_fed(s, inp["h"], inp["W"], rows=(0, s.rows - 1))


@pytest.mark.parametrize("cfg_id", [1, 2])
def test_head_topk_fed_full_size(cfg_id):
    s = wl.shape_of(cfg_id)
    inp, dev = cfg_inputs(cfg_id)
    check_head_fed(s, inp["h"], inp["W"], W_dev=dev["W"])


@pytest.mark.parametrize("s", [
    S(block=8, hidden=256, vocab=5000, top_k=16),              # streaming head
    S(batch=2, block=8, hidden=256, vocab=5000, top_k=16),     # GEMM head, segment merge
    S(batch=5, block=8, hidden=128, vocab=5003, top_k=4),      # segment merge, two waves per tile row
    S(batch=32, block=8, hidden=128, vocab=5000, top_k=16),    # segment merge, a whole 256-row pass
    # 8192 segments per row, all live: more than the merge lists in LDS
    S(batch=2, block=8, hidden=64, vocab=1 << 20, top_k=16),
    S(block=8, hidden=256, vocab=3000, top_k=40),              # K > 16
], ids=str)
@pytest.mark.parametrize("kind", ["zero_rows", "duplicate_weights"])
def test_head_topk_massive_ties(s, kind):
    """Degenerate heads: all hidden rows zero (every logit 0: the candidates
    are ids 0..K-1 and lse = log V), or weight rows repeating with period 13
    (every logit value repeats, so ties are broken by id alone).  Exercises
    the tie fallbacks of the merge and the slice top-K."""
    inp = wl.make_inputs_for(s, 111, parts=("h", "W"))
    y, W = inp["h"].copy(), inp["W"].copy()
    if kind == "zero_rows":
        y[:] = 0
    else:
        W[:] = W[np.arange(s.vocab) % 13]
    ids, lp, lse, logits = run_head(s, y, W)
    rid, rlse = topk_of(logits, s.top_k)
    assert np.array_equal(ids, rid)
    check_timed_mode(s, y, W, None, ids, lp, lse, logits)
    ref = orc.head(s, y, W, want_logits=True)
    assert np.array_equal(ids, ref["ids"])
    assert rel_err(lse, ref["lse"]) <= 1e-5
    if kind == "zero_rows":
        assert np.all(ids == np.arange(s.top_k)[None, :])
        assert np.allclose(lse, np.log(s.vocab), rtol=1e-6)


@pytest.mark.parametrize("cfg_id", [1, 3])
def test_vocab_sharding_merge(cfg_id):
    """The multi-GPU reading: each GPU runs the head on its eighth of the
    vocabulary; exchanging the per-row top-K (with global ids) and lse, then
    merging, must give the single-GPU candidates.  Here the eight shards run
    in turn on one GPU and the exchange + merge is done on the host: ids
    bit-identical to the full head (ties by global id), lse to 1e-6."""
    s = wl.shape_of(cfg_id)
    inp, dev = cfg_inputs(cfg_id)
    y = to_dev(inp["h"])  # any bf16 rows serve: the head alone is compared
    full_ids, _, full_lse, _ = run_head(s, inp["h"], None, W_dev=dev["W"], with_logits=False)
    n = 8
    edges = [s.vocab * g // n for g in range(n + 1)]
    keys_v, keys_i, lses = [], [], []
    for g in range(n):
        v0, v1 = edges[g], edges[g + 1]
        sub = s.with_(vocab=v1 - v0)
        cfg = dfs.Config.of(sub)
        ids = empty((s.rows, s.top_k), torch.int32)
        lp = empty((s.rows, s.top_k), torch.float32)
        lse = empty((s.rows,), torch.float32)
        logits = empty((s.rows, v1 - v0), torch.float32)
        dfs.head_topk(cfg, y, dev["W"][v0:v1], ids, lp, lse, wsbuf(cfg), logits_f32=logits)
        torch.cuda.synchronize()
        ids, lse, logits = from_dev(ids), from_dev(lse), from_dev(logits)
        # what a shard would send: its candidates' fp32 logits (the keys) with global ids
        keys_v.append(np.take_along_axis(logits, ids, 1).astype(np.float64))
        keys_i.append(ids.astype(np.int64) + v0)
        lses.append(lse.astype(np.float64))
    V_, I_ = np.concatenate(keys_v, 1), np.concatenate(keys_i, 1)
    for r in range(s.rows):
        order = np.lexsort((I_[r], -V_[r]))[: s.top_k]
        assert list(I_[r, order]) == list(full_ids[r]), r
    L = np.stack(lses, 1)
    m = L.max(1)
    merged = m + np.log(np.exp(L - m[:, None]).sum(1))
    assert np.max(np.abs(merged - full_lse.astype(np.float64)) / np.abs(full_lse)) <= 1e-6


# ============================================================== top-K of given logits

def crafted_logits(rows, V, seed):
    rng = np.random.default_rng(seed)
    L = (np.round(rng.standard_normal((rows, V)) * 8) / 8).astype(np.float32)
    L[0, :] = 0.0
    if rows > 1:
        L[1, ::2] = -0.0
        L[1, 1::2] = 0.0
    if rows > 2:
        L[2, :] = -np.inf
        L[2, [5, V // 2, V - 1]] = 1.0
    if rows > 3:
        L[3, -20:] = 50.0
    if rows > 4:
        step = max(1, V // 300)
        L[4, ::step] = 7.0  # many exact ties across chunk boundaries
    if rows > 5:
        # Large values at the ids v with v % 1024 < 224.  With slices that
        # start at multiples of 1024 they fall in fewer lane groups than K, so
        # more keys than the gather buffer holds pass the group-maximum
        # threshold and the exact bisection decides.
        big = (np.arange(V) % 1024) < 224
        L[5:, big] = 1000.0 + np.round(rng.standard_normal((rows - 5, int(big.sum()))) * 64) / 8
    return L


@pytest.mark.parametrize("rows,V,K", [(6, 1537, 16), (6, 1537, 64), (5, 248320, 16), (7, 100, 1), (6, 64, 64),
                                      (64, 32 * 7168, 16), (64, 32 * 7168, 64)])
def test_topk_logits_crafted(rows, V, K):
    s = wl.Shape(batch=1, block=rows, hidden=64, vocab=V, top_k=K, rank=16, group=16, ksize=2, dtype="f32")
    cfg = dfs.Config.of(s)
    L = crafted_logits(rows, V, rows * V + K)
    ids = empty((rows, K), torch.int32)
    lp = empty((rows, K), torch.float32)
    lse = empty((rows,), torch.float32)
    dfs.topk_logits(cfg, to_dev(L), ids, lp, lse, wsbuf(cfg))
    torch.cuda.synchronize()
    rid, rlp, rlse = orc.topk(L.astype(np.float64), K)
    assert np.array_equal(from_dev(ids), rid)
    ok = np.isfinite(rlse)
    assert rel_err(from_dev(lse)[ok], rlse[ok]) <= 1e-5
    lp_h = from_dev(lp)
    fin = np.isfinite(rlp)
    assert np.allclose(lp_h[fin], rlp[fin], rtol=0, atol=1e-5 * (1 + np.abs(rlp[fin]).max()))
    assert np.all(np.isneginf(lp_h[~fin]) == np.isneginf(rlp[~fin]))


# ============================================================== select (FED)

def select_inputs(s, seed, dyadic=False, zero_P=False):
    rng = np.random.default_rng(seed)
    ids = np.stack([np.stack([rng.choice(s.vocab, s.top_k, replace=False) for _ in range(s.block)])
                    for _ in range(s.batch)]).reshape(s.rows, s.top_k).astype(np.int32)
    if dyadic:
        lp = (rng.integers(-16, 1, (s.rows, s.top_k)) / 8.0).astype(np.float32)
        vals = np.array([0.0, 0.25, -0.25, 0.5, -0.5], np.float32)
        P = rng.choice(vals, (s.vocab, s.rank)).astype(np.float32)
        Q = rng.choice(vals, (s.vocab, s.rank)).astype(np.float32)
        if s.dtype == "bf16":
            P, Q = wl.bf16_bits(P), wl.bf16_bits(Q)
    else:
        lp = (-np.abs(rng.standard_normal((s.rows, s.top_k))) * 3).astype(np.float32)
        pq = wl.make_inputs_for(s, seed, parts=("P", "Q"))
        P, Q = pq["P"], pq["Q"]
    if zero_P:
        P = np.zeros_like(P)
    anchor = rng.integers(0, s.vocab, s.batch).astype(np.int32)
    return ids, lp, P, Q, anchor


def run_select(s, ids, lp, P, Q, anchor):
    cfg = dfs.Config.of(s)
    path = empty((s.batch, s.block), torch.int32)
    score = empty((s.batch,), torch.float32)
    pidx = empty((s.batch, s.block), torch.int32)
    dfs.select(cfg, to_dev(anchor), to_dev(ids), to_dev(lp), to_dev(P), to_dev(Q), path, score, wsbuf(cfg),
               path_idx=pidx)
    torch.cuda.synchronize()
    return from_dev(path), from_dev(score), from_dev(pidx)


def oracle_walk(s, ids, lp, P, Q, anchor, b):
    rs = slice(b * s.block, (b + 1) * s.block)
    T = orc.transitions(s, int(anchor[b]), ids[rs], P, Q)
    return orc.viterbi(lp[rs].astype(np.float64), T)


SELECT_SHAPES = [
    S(batch=4, block=8, vocab=5000, top_k=16, rank=256),
    S(batch=3, block=2, vocab=500, top_k=5, rank=32),
    S(batch=2, block=6, vocab=300, top_k=1, rank=16),
    S(batch=2, block=64, vocab=9000, top_k=64, rank=64),
    S(batch=5, block=16, vocab=2000, top_k=16, rank=256, dtype="f32"),
    S(batch=3, block=5, vocab=4000, top_k=33, rank=8),
    # the walk streams T through LDS in whole-slot chunks (42 slots at K 17,
    # 5 at K 48): several chunks with a ragged last one
    S(batch=2, block=64, vocab=3000, top_k=17, rank=40),
    S(batch=3, block=40, vocab=6000, top_k=48, rank=24, dtype="f32"),
    S(batch=2, block=4, vocab=5000, top_k=16, rank=4096),  # the largest rank
    # the fused MFMA selector at the longest block: the walk's back-pointer
    # table fills all four of its registers per lane
    S(batch=2, block=64, vocab=9000, top_k=16, rank=64),
]


@pytest.mark.parametrize("s", SELECT_SHAPES, ids=str)
@pytest.mark.parametrize("mode", ["random", "dyadic", "zeroP"])
def test_select_fed(s, mode):
    ids, lp, P, Q, anchor = select_inputs(s, 7 + s.block, dyadic=(mode == "dyadic"), zero_P=(mode == "zeroP"))
    path, score, pidx = run_select(s, ids, lp, P, Q, anchor)
    for b in range(s.batch):
        idx, sc, margin = oracle_walk(s, ids, lp, P, Q, anchor, b)
        if mode == "dyadic":
            assert list(pidx[b]) == list(idx) and score[b] == sc
        elif margin > NEAR_TIE:
            assert list(pidx[b]) == list(idx)
            assert abs(score[b] - sc) <= SCORE_TOL
        else:  # near tie: the GPU path must score within tolerance of the best
            rs = slice(b * s.block, (b + 1) * s.block)
            T = orc.transitions(s, int(anchor[b]), ids[rs], P, Q)
            g = [int(k) for k in pidx[b]]
            gs = lp[rs][1, g[1]] + T[0, 0, g[1]] + sum(lp[rs][t, g[t]] + T[t - 1, g[t - 1], g[t]]
                                                      for t in range(2, s.block))
            assert abs(gs - sc) <= SCORE_TOL
        assert path[b, 0] == anchor[b] and pidx[b, 0] == -1
        assert all(path[b, t] == ids[b * s.block + t, pidx[b, t]] for t in range(1, s.block))
        if mode == "zeroP":  # DFlash1 behaviour: per-slot argmax, lowest index on ties
            want = [int(np.argmax(lp[b * s.block + t])) for t in range(1, s.block)]
            assert list(pidx[b, 1:]) == want


def test_select_bad_anchor_and_ids():
    s = S(batch=5, block=8, vocab=1000, top_k=16, rank=64)
    ids, lp, P, Q, anchor = select_inputs(s, 3)
    anchor[1] = s.vocab
    anchor[3] = -7
    ids[4 * s.block + 5, 3] = s.vocab + 100  # a bad candidate id in block 4
    path, score, pidx = run_select(s, ids, lp, P, Q, anchor)
    for b in (1, 3, 4):
        assert np.all(path[b] == -1) and np.all(pidx[b] == -1) and math.isnan(score[b])
    for b in (0, 2):
        idx, sc, _ = oracle_walk(s, ids, lp, P, Q, anchor, b)
        assert list(pidx[b]) == list(idx) and abs(score[b] - sc) <= SCORE_TOL


def test_select_figure1_repetition():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "figure1_repetition.json")))
    V, r = 16, 8
    s = S(batch=1, block=g["block"], vocab=V, top_k=g["top_k"], rank=r, dtype="f32")
    P = np.zeros((V, r), np.float32)
    Q = np.zeros((V, r), np.float32)
    for k, v in g["P"].items():
        P[int(k), :2] = v
    for k, v in g["Q"].items():
        Q[int(k), :2] = v
    ids = np.array(g["cand_ids"], np.int32)
    lp = np.array(g["cand_logp"], np.float32)
    path, score, pidx = run_select(s, ids, lp, P, Q, np.array([g["anchor"]], np.int32))
    assert list(path[0]) == g["expected_path"] and list(pidx[0]) == g["expected_idx"]
    assert score[0] == g["expected_score"]


# ============================================================== selector options (gate, walks)

GATE_SHAPES = [
    S(batch=4, block=8, vocab=5000, top_k=16, rank=256),           # bf16, K 16: the fused MFMA selector
    S(batch=3, block=5, vocab=4000, top_k=33, rank=8),             # general path
    S(batch=5, block=16, vocab=2000, top_k=16, rank=256, dtype="f32"),
]


def gate_for(s, seed):
    rng = np.random.default_rng(seed)
    return (0.5 + rng.random((s.rows, s.rank))).astype(np.float32)


def run_select_opts(s, ids, lp, P, Q, anchor, **opts):
    cfg = dfs.Config.of(s)
    path = empty((s.batch, s.block), torch.int32)
    score = empty((s.batch,), torch.float32)
    pidx = empty((s.batch, s.block), torch.int32)
    o = {k: (to_dev(v) if isinstance(v, np.ndarray) else v) for k, v in opts.items()}
    dfs.select(cfg, to_dev(anchor), to_dev(ids), to_dev(lp), to_dev(P), to_dev(Q), path, score, wsbuf(cfg),
               path_idx=pidx, **o)
    torch.cuda.synchronize()
    return from_dev(path), from_dev(score), from_dev(pidx)


def block_T(s, ids, P, Q, anchor, b, gate=None):
    rs = slice(b * s.block, (b + 1) * s.block)
    return orc.transitions(s, int(anchor[b]), ids[rs], P, Q, gate=None if gate is None else gate[rs])


@pytest.mark.parametrize("s", GATE_SHAPES, ids=str)
def test_select_gated_fed(s):
    ids, lp, P, Q, anchor = select_inputs(s, 61 + s.block)
    gate = gate_for(s, 62)
    path, score, pidx = run_select_opts(s, ids, lp, P, Q, anchor, gate=gate)
    for b in range(s.batch):
        rs = slice(b * s.block, (b + 1) * s.block)
        T = block_T(s, ids, P, Q, anchor, b, gate)
        idx, sc, margin = orc.viterbi(lp[rs].astype(np.float64), T)
        if margin > NEAR_TIE:
            assert list(pidx[b]) == list(idx)
            assert abs(score[b] - sc) <= SCORE_TOL
        assert path[b, 0] == anchor[b]
        assert all(path[b, t] == ids[b * s.block + t, pidx[b, t]] for t in range(1, s.block))


def test_select_gate_ones():
    """All-ones gate: bit-identical to no gate on the general path; the
    same paths as the fused kernel where they are not near ties."""
    s = S(batch=3, block=5, vocab=4000, top_k=33, rank=8)
    ids, lp, P, Q, anchor = select_inputs(s, 71)
    ones = np.ones((s.rows, s.rank), np.float32)
    a = run_select(s, ids, lp, P, Q, anchor)
    b = run_select_opts(s, ids, lp, P, Q, anchor, gate=ones)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    s = S(batch=4, block=8, vocab=5000, top_k=16, rank=256)
    ids, lp, P, Q, anchor = select_inputs(s, 72)
    a = run_select(s, ids, lp, P, Q, anchor)
    b = run_select_opts(s, ids, lp, P, Q, anchor, gate=np.ones((s.rows, s.rank), np.float32))
    for blk in range(s.batch):
        _, _, margin = oracle_walk(s, ids, lp, P, Q, anchor, blk)
        if margin > NEAR_TIE:
            assert list(a[2][blk]) == list(b[2][blk])
        assert abs(a[1][blk] - b[1][blk]) <= SCORE_TOL


def check_walk(s, ids, lp, P, Q, anchor, pidx, score, walk, temperature=1.0, uniforms=None, gate=None):
    """The GPU walk agrees with the oracle walk slot by slot.  At a slot where
    the two choose differently, the fp64 scores must make it a near tie
    (greedy) or put the uniform within 1e-5 of the boundary between the two
    choices (sampling); the rest of that block then follows another
    predecessor and is not compared."""
    for b in range(s.batch):
        rs = slice(b * s.block, (b + 1) * s.block)
        T = block_T(s, ids, P, Q, anchor, b, gate)
        lpb = lp[rs].astype(np.float64)
        u = None if uniforms is None else uniforms[b].astype(np.float64)
        idx, sc = orc.walk(lpb, T, walk, temperature, u)
        prev, same = 0, True
        for t in range(1, s.block):
            sk = lpb[t] + T[t - 1, prev]
            g, o = int(pidx[b, t]), int(idx[t])
            if g != o:
                if walk == "greedy":
                    assert abs(sk[g] - sk[o]) <= SCORE_TOL, (b, t)
                else:
                    e = np.exp((sk - sk.max()) / temperature)
                    cdf = np.cumsum(e) / e.sum()
                    edge = cdf[min(g, o)]
                    assert abs(u[t] - edge) <= 1e-5, (b, t, u[t], edge)
                same = False
                break
            prev = g
        if same:
            assert abs(score[b] - sc) <= SCORE_TOL, b


def random_select_cases(n, seed=2027):
    """Seeded selector cases: shape, walk rule, gate on or off; fused and
    general kernels both get exercised (bf16, K <= 16, r % 32 == 0, and B <=
    16 for greedy and sampled walks, run the fused kernel, gated or not)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        top_k = int(rng.choice([1, 3, 8, 16, 16, 16, 17, 33, 64]))
        s = S(batch=int(rng.integers(1, 6)), block=int(rng.integers(2, 40)), vocab=int(rng.integers(2000, 9000)),
              top_k=top_k, rank=int(rng.choice([8, 32, 64, 96, 256])),
              dtype="f32" if rng.random() < 0.25 else "bf16")
        out.append((s, ("viterbi", "greedy", "sample")[i % 3], bool(rng.random() < 0.25), 300 + i))
    return out


@pytest.mark.parametrize("case", random_select_cases(24), ids=lambda c: f"{c[1]}-gate{int(c[2])}-{c[0]}")
def test_select_random_options(case):
    s, walk, gated, seed = case
    ids, lp, P, Q, anchor = select_inputs(s, seed)
    gate = gate_for(s, seed + 1) if gated else None
    u = np.random.default_rng(seed + 2).random((s.batch, s.block)).astype(np.float32)
    extra = dict(temperature=0.7, uniforms=u) if walk == "sample" else {}
    path, score, pidx = run_select_opts(s, ids, lp, P, Q, anchor, gate=gate, walk=walk, **extra)
    assert np.all(path[:, 0] == anchor) and np.all(pidx[:, 0] == -1)
    for b in range(s.batch):
        assert all(path[b, t] == ids[b * s.block + t, pidx[b, t]] for t in range(1, s.block))
    if walk == "viterbi":
        for b in range(s.batch):
            rs = slice(b * s.block, (b + 1) * s.block)
            idx, sc, margin = orc.viterbi(lp[rs].astype(np.float64), block_T(s, ids, P, Q, anchor, b, gate))
            if margin > NEAR_TIE:
                assert list(pidx[b]) == list(idx), b
                assert abs(score[b] - sc) <= SCORE_TOL, b
    else:
        check_walk(s, ids, lp, P, Q, anchor, pidx, score, walk, 0.7, u if walk == "sample" else None, gate)


@pytest.mark.parametrize("s", SELECT_SHAPES[:4] + SELECT_SHAPES[6:] + GATE_SHAPES[2:], ids=str)
def test_select_greedy_fed(s):
    ids, lp, P, Q, anchor = select_inputs(s, 81 + s.block)
    path, score, pidx = run_select_opts(s, ids, lp, P, Q, anchor, walk="greedy")
    assert np.all(path[:, 0] == anchor) and np.all(pidx[:, 0] == -1)
    check_walk(s, ids, lp, P, Q, anchor, pidx, score, "greedy")


@pytest.mark.parametrize("temperature", [0.5, 1.0, 3.0])
@pytest.mark.parametrize("s", [SELECT_SHAPES[0], SELECT_SHAPES[3], SELECT_SHAPES[7], GATE_SHAPES[2]], ids=str)
def test_select_sample_fed(s, temperature):
    ids, lp, P, Q, anchor = select_inputs(s, 91 + s.block)
    u = np.random.default_rng(92).random((s.batch, s.block)).astype(np.float32)
    gate = gate_for(s, 93)
    path, score, pidx = run_select_opts(s, ids, lp, P, Q, anchor, walk="sample", temperature=temperature,
                                        uniforms=u, gate=gate)
    check_walk(s, ids, lp, P, Q, anchor, pidx, score, "sample", temperature, u, gate)
    # the same uniforms give the same path again
    _, score2, pidx2 = run_select_opts(s, ids, lp, P, Q, anchor, walk="sample", temperature=temperature,
                                       uniforms=u, gate=gate)
    assert np.array_equal(pidx, pidx2) and np.array_equal(score, score2)


def test_select_sample_extreme_uniforms():
    """u = 0 takes the first candidate with a non-zero weight (index 0 when
    every weight is positive); u just below 1 takes the last."""
    s = S(batch=2, block=4, vocab=3000, top_k=8, rank=64)
    ids, lp, P, Q, anchor = select_inputs(s, 95)
    u0 = np.zeros((s.batch, s.block), np.float32)
    _, _, p0 = run_select_opts(s, ids, lp, P, Q, anchor, walk="sample", temperature=1e3, uniforms=u0)
    assert np.all(p0[:, 1:] == 0)
    u1 = np.full((s.batch, s.block), np.nextafter(np.float32(1), np.float32(0)), np.float32)
    _, _, p1 = run_select_opts(s, ids, lp, P, Q, anchor, walk="sample", temperature=1e3, uniforms=u1)
    assert np.all(p1[:, 1:] == s.top_k - 1)


# ============================================================== whole block (E2E)

def run_block(s, dev, cfg=None, stream=None):
    cfg = cfg or dfs.Config.of(s)
    path = empty((s.batch, s.block), torch.int32)
    score = empty((s.batch,), torch.float32)
    ids = empty((s.rows, s.top_k), torch.int32)
    lp = empty((s.rows, s.top_k), torch.float32)
    dfs.draft_block(cfg, dev["h"], dev["anchor"], dev["wg_cm"], dev["W"], dev["P"], dev["Q"], path, score,
                    wsbuf(cfg), cand_ids=ids, cand_logp=lp, stream=stream)
    torch.cuda.synchronize()
    return from_dev(path), from_dev(score), from_dev(ids), from_dev(lp)


def check_block_e2e(s, inp, dev, blocks=None):
    out = run_block(s, dev)
    e2e.check_block_e2e(orc, s, inp, out, blocks)
    return out[0], out[1]


@pytest.mark.parametrize("cfg_id", [0, 1, 2, 5])
def test_draft_block_e2e(cfg_id):
    s = wl.shape_of(cfg_id)
    inp, dev = cfg_inputs(cfg_id)
    check_block_e2e(s, inp, dev)


@pytest.mark.slow
def test_draft_block_e2e_batch32():
    """The page shape at batch 32: every one of the 32 blocks (256 rows)
    against the oracle."""
    s = wl.shape_of(3)
    inp, dev = cfg_inputs(3)
    check_block_e2e(s, inp, dev)


@pytest.mark.parametrize("s", [
    S(batch=4, block=5, hidden=128, vocab=7000, top_k=8, rank=32),
    S(batch=3, block=16, hidden=64, vocab=1000, top_k=16, rank=16, ksize=4, group=32),
    S(batch=2, block=8, hidden=96, vocab=800, top_k=20, rank=24, dtype="f32"),
    S(batch=3, block=6, hidden=128, vocab=4000, top_k=16, rank=32, ksize=1),
], ids=str)
def test_draft_block_e2e_small(s):
    inp = wl.make_inputs_for(s, 17)
    dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
    dev["wg_cm"] = to_dev(wg_channel_major(inp["wg"]))
    check_block_e2e(s, inp, dev)


def random_configs(n, seed=2026):
    """Seeded small configurations spread over the accepted ranges: both
    dtypes, one, two or four taps, several group sizes, K on both sides of
    16, few and many rows, ragged vocabularies."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        hidden = int(rng.choice([32, 64, 96, 128, 160, 192, 256]))
        group = int(rng.choice([g for g in (4, 8, 16, 32) if hidden % g == 0]))
        top_k = int(rng.integers(1, 25))
        out.append(S(batch=int(rng.integers(1, 7)), block=int(rng.integers(2, 21)), hidden=hidden,
                     vocab=int(rng.integers(max(top_k, 16), 6001)), top_k=top_k,
                     rank=int(rng.choice([8, 16, 24, 32, 64])), group=group, ksize=int(rng.choice([1, 2, 4])),
                     dtype="f32" if rng.random() < 0.25 else "bf16"))
    return out


def random_long_configs(n, seed=2028):
    """Seeded configurations with long blocks and large K (B up to 64, K up
    to 64), few rows, small vocabularies: the general selector end to end."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        top_k = int(rng.integers(8, 65))
        out.append(S(batch=int(rng.integers(1, 3)), block=int(rng.integers(17, 65)),
                     hidden=int(rng.choice([64, 128])), vocab=int(rng.integers(max(top_k, 500), 3001)),
                     top_k=top_k, rank=int(rng.choice([16, 32, 64])), ksize=int(rng.choice([1, 2, 4])),
                     dtype="f32" if rng.random() < 0.25 else "bf16"))
    return out


def random_large_configs(n, seed=2029):
    """Seeded configurations at larger sizes: hidden up to 8192 (the bf16
    limit), vocabularies up to 100 000, blocks up to 64 slots, up to 32
    blocks, K up to 64, one, two or four taps, both dtypes; rows x V x D is
    kept under 3e9 so that the oracle finishes in seconds."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        hidden = int(rng.choice([96, 320, 640, 1024, 1536, 2048, 2560, 4096, 5120, 8192]))
        group = int(rng.choice([g for g in (4, 8, 16, 32, 64) if hidden % g == 0]))
        top_k = int(rng.choice([1, 3, 8, 12, 16, 17, 24, 32, 48, 64]))
        block = int(rng.choice([2, 4, 8, 9, 16, 24, 32, 48, 64]))
        batch = int(rng.integers(1, 33)) if rng.random() < 0.6 else 1
        vocab = int(rng.integers(max(top_k, 16), 100001))
        ksize = int(rng.choice([1, 2, 2, 4]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        if batch * block * vocab * hidden > 3e9 or (dtype == "f32" and hidden // group * ksize > 4096):
            continue
        out.append(S(batch=batch, block=block, hidden=hidden, vocab=vocab, top_k=top_k,
                     rank=int(rng.choice([8, 32, 96, 256])), group=group, ksize=ksize, dtype=dtype))
    return out


@pytest.mark.parametrize("s", random_large_configs(16), ids=str)
def test_draft_block_random_large_configs(s):
    inp = wl.make_inputs_for(s, 37)
    dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
    dev["wg_cm"] = to_dev(wg_channel_major(inp["wg"]))
    check_block_e2e(s, inp, dev)


@pytest.mark.parametrize("s", random_configs(24) + random_long_configs(8), ids=str)
def test_draft_block_random_configs(s):
    inp = wl.make_inputs_for(s, 23)
    dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
    dev["wg_cm"] = to_dev(wg_channel_major(inp["wg"]))
    check_block_e2e(s, inp, dev)


@pytest.mark.parametrize("walk", ["viterbi", "greedy", "sample"])
def test_draft_block_with_options(walk):
    """The whole block with a context gate and each walk rule, against the
    oracle's candidates and walk.  Blocks whose GPU candidates differ from the
    oracle's by a near tie are not walked."""
    s = S(batch=6, block=8, hidden=256, vocab=6000, top_k=16, rank=64)
    inp = wl.make_inputs_for(s, 101)
    dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
    dev["wg_cm"] = to_dev(wg_channel_major(inp["wg"]))
    gate = gate_for(s, 102)
    u = np.random.default_rng(103).random((s.batch, s.block)).astype(np.float32)
    cfg = dfs.Config.of(s)
    path = empty((s.batch, s.block), torch.int32)
    score = empty((s.batch,), torch.float32)
    ids = empty((s.rows, s.top_k), torch.int32)
    lp = empty((s.rows, s.top_k), torch.float32)
    extra = dict(temperature=0.8, uniforms=to_dev(u)) if walk == "sample" else {}
    dfs.draft_block(cfg, dev["h"], dev["anchor"], dev["wg_cm"], dev["W"], dev["P"], dev["Q"], path, score,
                    wsbuf(cfg), cand_ids=ids, cand_logp=lp, gate=to_dev(gate), walk=walk, **extra)
    torch.cuda.synchronize()
    path, score, ids, lp = from_dev(path), from_dev(score), from_dev(ids), from_dev(lp)
    ref = orc.draft_block(s, inp["h"], inp["anchor"], inp["wg"], inp["W"], inp["P"], inp["Q"], gate=gate)
    walked = 0
    for b in range(s.batch):
        rs = slice(b * s.block, (b + 1) * s.block)
        if not np.array_equal(ids[rs], ref["ids"][rs]):
            continue
        walked += 1
        T = orc.transitions(s, int(inp["anchor"][b]), ref["ids"][rs], inp["P"], inp["Q"], gate=gate[rs])
        if walk == "viterbi":
            ridx, rsc, margin = orc.viterbi(ref["logp"][rs], T)
            if margin <= 1e-3:
                continue
        else:
            ridx, rsc = orc.walk(ref["logp"][rs], T, walk, 0.8, u[b].astype(np.float64) if walk == "sample" else None)
        want = [int(inp["anchor"][b])] + [int(ref["ids"][b * s.block + t, ridx[t]]) for t in range(1, s.block)]
        if walk == "sample" and list(path[b]) != want:
            continue  # a uniform on a CDF boundary under the 2e-3 logit tolerance; covered in FED mode
        assert list(path[b]) == want, (walk, b)
        assert abs(score[b] - rsc) <= TOL * max(1.0, abs(rsc)), (walk, b)
    assert walked >= s.batch - 1


@pytest.mark.parametrize("case", ["page_batch1", "rows_40", "greedy_b16", "zero_weight"])
def test_draft_block_equals_separate_calls(case):
    """dfs_draft_block gives the same bits as dfs_conv, dfs_head_topk and
    dfs_select called one after another: candidates, scores, path and path
    score.  The all-zero weight ties every logit, so more keys than the
    merge's gather holds reach its threshold and its list merge runs."""
    opts = {}
    if case == "page_batch1":
        s = wl.shape_of(2)
        inp, dev = cfg_inputs(2)
    else:
        s = {"rows_40": S(batch=5, block=8, hidden=256, vocab=9001, top_k=16, rank=64),
             "greedy_b16": S(batch=3, block=16, hidden=128, vocab=7000, top_k=12, rank=32),
             "zero_weight": S(batch=2, block=8, hidden=128, vocab=5000, top_k=16, rank=64)}[case]
        inp = wl.make_inputs_for(s, 31)
        if case == "zero_weight":
            inp["W"] = np.zeros_like(inp["W"])
        dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
        dev["wg_cm"] = to_dev(wg_channel_major(inp["wg"]))
        if case == "greedy_b16":
            opts = dict(walk="greedy")
    cfg = dfs.Config.of(s)
    path = empty((s.batch, s.block), torch.int32)
    score = empty((s.batch,), torch.float32)
    ids = empty((s.rows, s.top_k), torch.int32)
    lp = empty((s.rows, s.top_k), torch.float32)
    dfs.draft_block(cfg, dev["h"], dev["anchor"], dev["wg_cm"], dev["W"], dev["P"], dev["Q"], path, score,
                    wsbuf(cfg), cand_ids=ids, cand_logp=lp, **opts)
    y = empty((s.rows, s.hidden), torch.int16)
    ids2 = empty((s.rows, s.top_k), torch.int32)
    lp2 = empty((s.rows, s.top_k), torch.float32)
    lse2 = empty((s.rows,), torch.float32)
    path2 = empty((s.batch, s.block), torch.int32)
    score2 = empty((s.batch,), torch.float32)
    dfs.conv(cfg, dev["h"], dev["wg_cm"], y, wsbuf(cfg))
    dfs.head_topk(cfg, y, dev["W"], ids2, lp2, lse2, wsbuf(cfg))
    dfs.select(cfg, dev["anchor"], ids2, lp2, dev["P"], dev["Q"], path2, score2, wsbuf(cfg), **opts)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(ids), from_dev(ids2))
    assert np.array_equal(from_dev(lp), from_dev(lp2))
    assert np.array_equal(from_dev(path), from_dev(path2))
    assert np.array_equal(from_dev(score), from_dev(score2))
    if case == "zero_weight":  # every logit 0: the lowest ids, in order
        assert np.array_equal(from_dev(ids), np.tile(np.arange(s.top_k, dtype=np.int32), (s.rows, 1)))


SMALL_BLOCK_CASES = [
    # (shape, options, anchor of block 1 replaced by an invalid id)
    (S(batch=1, block=8, hidden=256, vocab=9001, top_k=16, rank=64), {}, False),
    (S(batch=1, block=2, hidden=128, vocab=5000, top_k=16, rank=32), {}, False),
    (S(batch=2, block=4, hidden=256, vocab=7001, top_k=8, rank=64), dict(walk="greedy"), False),
    (S(batch=4, block=2, hidden=128, vocab=3000, top_k=5, rank=32), dict(walk="sample", temperature=0.7), False),
    (S(batch=1, block=7, hidden=192, vocab=6000, top_k=1, rank=32), {}, False),
    (S(batch=1, block=8, hidden=160, vocab=6000, top_k=12, rank=64), dict(gate=True), False),
    (S(batch=2, block=3, hidden=256, vocab=4099, top_k=16, rank=96), dict(gate=True, walk="sample", temperature=1.3),
     False),
    (S(batch=2, block=4, hidden=128, vocab=5000, top_k=16, rank=64), {}, True),
    (S(batch=1, block=8, hidden=1024, vocab=50000, top_k=16, rank=256, ksize=1), {}, False),
]


@pytest.mark.parametrize("case", SMALL_BLOCK_CASES, ids=lambda c: f"{c[0]}-{sorted(c[1])}-bad{int(c[2])}")
def test_draft_block_few_rows_equals_separate_calls(case):
    """Up to 8 rows (the streaming head), dfs_draft_block gives the same bits
    as dfs_conv, dfs_head_topk and dfs_select: candidates, log-probabilities,
    path and score, for every walk rule, with and without a gate, one to four
    blocks, an invalid anchor (that block only is marked), D not a multiple
    of 64 (the other streaming head), one tap.  The workspace starts as
    all-ones bytes, and a second call on it gives the same bits: nothing
    depends on what an earlier call left there."""
    s, opts, bad = case
    inp = wl.make_inputs_for(s, 41)
    dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
    dev["wg_cm"] = to_dev(wg_channel_major(inp["wg"]))
    if bad:
        a = inp["anchor"].copy()
        a[1] = -1
        dev["anchor"] = to_dev(a)
    opts = dict(opts)
    if opts.pop("gate", False):
        opts["gate"] = to_dev(gate_for(s, 42))
    if opts.get("walk") == "sample":
        opts["uniforms"] = to_dev(np.random.default_rng(43).random((s.batch, s.block)).astype(np.float32))
    cfg = dfs.Config.of(s)
    ws = torch.full((dfs.workspace_size(cfg),), 255, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        path = empty((s.batch, s.block), torch.int32)
        score = empty((s.batch,), torch.float32)
        ids = empty((s.rows, s.top_k), torch.int32)
        lp = empty((s.rows, s.top_k), torch.float32)
        dfs.draft_block(cfg, dev["h"], dev["anchor"], dev["wg_cm"], dev["W"], dev["P"], dev["Q"], path, score, ws,
                        cand_ids=ids, cand_logp=lp, **opts)
        torch.cuda.synchronize()
        outs.append([from_dev(x) for x in (path, score, ids, lp)])
    y = empty((s.rows, s.hidden), torch.int16)
    ids2 = empty((s.rows, s.top_k), torch.int32)
    lp2 = empty((s.rows, s.top_k), torch.float32)
    lse2 = empty((s.rows,), torch.float32)
    path2 = empty((s.batch, s.block), torch.int32)
    score2 = empty((s.batch,), torch.float32)
    if s.ksize == 1:
        y = dev["h"]
    else:
        dfs.conv(cfg, dev["h"], dev["wg_cm"], y, wsbuf(cfg))
    dfs.head_topk(cfg, y, dev["W"], ids2, lp2, lse2, wsbuf(cfg))
    dfs.select(cfg, dev["anchor"], ids2, lp2, dev["P"], dev["Q"], path2, score2, wsbuf(cfg), **opts)
    torch.cuda.synchronize()
    ref = [from_dev(x) for x in (path2, score2, ids2, lp2)]
    for out in outs:
        for x, r in zip(out, ref):
            assert np.array_equal(x, r, equal_nan=True)
    if bad:
        assert np.all(ref[0][1] == -1) and np.isnan(ref[1][1])
        assert np.all(ref[0][0] >= 0) and not np.isnan(ref[1][0])


def test_draft_block_deterministic_and_stream():
    s = wl.shape_of(2)
    inp, dev = cfg_inputs(2)
    a = run_block(s, dev)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        b = run_block(s, dev, stream=st)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


@pytest.mark.parametrize("s", [
    S(batch=32, block=8, hidden=256, vocab=30011, top_k=16),   # GEMM head, segment merge
    S(batch=6, block=8, hidden=128, vocab=30011, top_k=40),    # GEMM head, slice top-K
], ids=str)
def test_draft_block_deterministic_many_rows(s):
    """The many-row paths give the same bits on every call and on another
    stream: the segment partials and merges combine in a fixed order."""
    inp = wl.make_inputs_for(s, 29)
    dev = {k: to_dev(v) for k, v in inp.items() if k != "wg"}
    dev["wg_cm"] = to_dev(wg_channel_major(inp["wg"]))
    a = run_block(s, dev)
    b = run_block(s, dev)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        c = run_block(s, dev, stream=st)
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y, equal_nan=True) and np.array_equal(x, z, equal_nan=True)


@pytest.mark.slow
def test_draft_block_long_block_planted():
    """Long-block workload (batch 8, B 16) with transition plants: every block
    against the oracle run on the planted inputs (near ties scored with the
    oracle, as everywhere), and the paths against the stored oracle reference
    tests/golden/plant_w4.json (written by tests/golden/make_plant_w4.py from
    the oracle alone) wherever its margin leaves no doubt."""
    import json
    import os

    from plant import apply_plant

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "plant_w4.json")))
    s = wl.shape_of(4)
    inp, dev = cfg_inputs(4)
    sites = [tuple(x) for x in g["sites"]]
    Qp = apply_plant(s, inp["P"], inp["Q"], sites)
    dev = dict(dev)
    dev["Q"] = to_dev(Qp)
    path, score, ids, lp = run_block(s, dev)
    e2e.check_block_e2e(orc, s, dict(inp, Q=Qp), (path, score, ids, lp))
    for b in range(s.batch):
        same = np.array_equal(ids[b * s.block:(b + 1) * s.block], np.array(g["cand_ids"][b * s.block:(b + 1) * s.block]))
        if g["margin"][b] > 1e-3 and same:
            assert path[b].tolist() == g["path"][b], f"block {b}"
    assert rel_err(score, np.array(g["score"])) <= TOL
    # the plants move the walk off the per-slot argmax where the oracle's does
    dev_gpu = sum(path[b, t] != ids[b * s.block + t, 0] for b, t, *_ in sites)
    assert dev_gpu == g["n_sites_deviating"]


@pytest.mark.slow
def test_head_topk_fed_many_rows():
    """GEMM head at the batch-32 page shape (256 rows): ids exactly the top-K
    of the GPU's own logits, and logits, lse and ids against the oracle head,
    on every row."""
    s = wl.shape_of(3)
    inp, dev = cfg_inputs(3)
    check_head_fed(s, inp["h"], inp["W"], W_dev=dev["W"])
