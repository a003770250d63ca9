"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test ties one oracle step to a closed form, an invariant, a library
routine (numpy matmul, lexsort, scipy logsumexp), brute-force enumeration, or
the hand-derived repetition example of the Inco AI post (Figure 1), so that a
dropped term, a wrong sign or index, or a transposed operand fails a test.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_shape(**kw):
    base = dict(batch=2, block=4, hidden=64, vocab=300, top_k=4, rank=16, group=16, ksize=2, dtype="f32")
    base.update(kw)
    return wl.Shape(**base)


def rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


# --------------------------------------------------------------------------- conv

def test_conv_zero_generator_is_two_tap_mean(orc):
    # Wg = 0 => both taps have logit 0 => weights 1/2 each:
    # y[t] = (h[t] + h[t-1]) / 2 inside a block, y[0] = h[0] / 2 at its start.
    s = f32_shape()
    h = rand((s.rows, s.hidden), 1)
    wg = np.zeros((s.hidden, s.groups * s.ksize), np.float32)
    z, w, y = orc.conv(s, h, wg)
    assert np.all(z == 0.0) and np.all(w == 0.5)
    hd = h.astype(np.float64)
    for b in range(s.batch):
        r0 = b * s.block
        assert np.array_equal(y[r0], 0.5 * hd[r0])
        for t in range(1, s.block):
            assert np.array_equal(y[r0 + t], 0.5 * (hd[r0 + t] + hd[r0 + t - 1]))


@pytest.mark.parametrize("sign", [+1, -1])
def test_conv_saturated_taps(orc, sign):
    # Channel 0 of h is a constant 1 and row 0 of Wg gives tap 0 a logit of
    # +-40 over tap 1: the softmax saturates, so y[t] = h[t] (sign +1) or
    # y[t] = h[t-1] with y[0] = 0 (sign -1), to within e^-40.
    s = f32_shape()
    h = rand((s.rows, s.hidden), 2)
    h[:, 0] = 1.0
    wg = np.zeros((s.hidden, s.groups * s.ksize), np.float32)
    wg[0, 0::2] = 40.0 * sign
    _, _, y = orc.conv(s, h, wg)
    hd = h.astype(np.float64)
    for b in range(s.batch):
        r0 = b * s.block
        for t in range(s.block):
            if sign > 0:
                want = hd[r0 + t]
            else:
                want = hd[r0 + t - 1] if t > 0 else np.zeros(s.hidden)
            np.testing.assert_allclose(y[r0 + t], want, rtol=0, atol=1e-15)


def test_conv_unit_generator_closed_form(orc):
    # Column g*ks+j of Wg is the unit vector of channel c(g, j), so the tap
    # logits are h[t, c(g, j)] and the weights are the logistic function of
    # their difference.  Pins the group-major column order g*ks + j.
    s = f32_shape(batch=1, block=3, hidden=32, group=16)
    h = rand((s.rows, s.hidden), 3)
    G = s.groups
    pick = {(0, 0): 5, (0, 1): 20, (1, 0): 31, (1, 1): 2}
    wg = np.zeros((s.hidden, G * 2), np.float32)
    for (g, j), c in pick.items():
        wg[c, g * 2 + j] = 1.0
    z, w, y = orc.conv(s, h, wg)
    for t in range(s.block):
        for g in range(G):
            a, b = float(h[t, pick[(g, 0)]]), float(h[t, pick[(g, 1)]])
            w0 = 1.0 / (1.0 + math.exp(b - a))
            assert z[t, 2 * g] == a and z[t, 2 * g + 1] == b
            assert abs(w[t, 2 * g] - w0) < 1e-15 and abs(w[t, 2 * g + 1] - (1.0 - w0)) < 1e-15
            for c in range(g * 16, (g + 1) * 16):
                want = w0 * float(h[t, c]) + ((1.0 - w0) * float(h[t - 1, c]) if t > 0 else 0.0)
                assert abs(y[t, c] - want) < 1e-14


def test_conv_single_tap_is_identity(orc):
    s = f32_shape(ksize=1)
    h = rand((s.rows, s.hidden), 4)
    wg = rand((s.hidden, s.groups), 5)
    _, w, y = orc.conv(s, h, wg)
    assert np.all(w == 1.0)
    assert np.array_equal(y, h.astype(np.float64))


def test_conv_tap_weights_sum_to_one_and_positive(orc):
    s = f32_shape(ksize=4, group=8)
    h = rand((s.rows, s.hidden), 6)
    wg = rand((s.hidden, s.groups * 4), 7, 0.5)
    _, w, _ = orc.conv(s, h, wg)
    sums = w.reshape(s.rows, s.groups, 4).sum(-1)
    np.testing.assert_allclose(sums, 1.0, atol=1e-15)
    assert np.all(w > 0)


def test_conv_channel_permutation_within_group_commutes(orc):
    s = f32_shape()
    h = rand((s.rows, s.hidden), 8)
    wg = rand((s.hidden, s.groups * s.ksize), 9, 1 / 8)
    rng = np.random.default_rng(10)
    perm = np.concatenate([g * 16 + rng.permutation(16) for g in range(s.groups)])
    _, _, y = orc.conv(s, h, wg)
    _, _, yp = orc.conv(s, np.ascontiguousarray(h[:, perm]), np.ascontiguousarray(wg[perm]))
    np.testing.assert_allclose(yp, y[:, perm], rtol=0, atol=1e-13)


def test_conv_causal_and_block_local(orc):
    s = f32_shape(batch=3)
    h = rand((s.rows, s.hidden), 11)
    wg = rand((s.hidden, s.groups * s.ksize), 12, 1 / 8)
    _, _, y = orc.conv(s, h, wg)
    # changing position t of block 1 leaves earlier positions and other blocks unchanged
    h2 = h.copy()
    t = 2
    h2[s.block + t] += 1.0
    _, _, y2 = orc.conv(s, h2, wg)
    changed = np.any(y2 != y, axis=1)
    want = np.zeros(s.rows, bool)
    want[s.block + t] = True
    want[s.block + t + 1] = True  # ks = 2: the next position reads h[t]
    assert np.array_equal(changed, want)
    # each block equals the conv of that block alone
    for b in range(s.batch):
        sl = slice(b * s.block, (b + 1) * s.block)
        _, _, yb = orc.conv(s.with_(batch=1), np.ascontiguousarray(h[sl]), wg)
        assert np.array_equal(yb, y[sl])


def test_bf16_rounding_is_round_to_nearest_even(orc):
    s = f32_shape(dtype="bf16")
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-30, -(1 + 2**-8), 0.0, -0.0,
                  2**-130, 3.0e38, 1 - 2**-9, 3 * 2**-134, 5 * 2**-134], dtype=np.float64)
    got = orc.round_to(s, x)
    # 2**-130 is a bf16 subnormal (exact, mantissa bit 3); subnormal spacing is
    # 2**-133, so 1.5 and 2.5 spacings round to the even multiples 2 and 2.
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x0000, 0x8000, 0x0008, 0x7F62, 0x3F80,
            0x0002, 0x0002]
    assert [int(v) for v in got] == want
    # on values exact in fp32 the result equals the fp32 -> bf16 generator path
    v = rand(4096, 13, 3.0).astype(np.float64)
    assert np.array_equal(orc.round_to(s, v), wl.bf16_bits(v.astype(np.float32)))


# --------------------------------------------------------------------------- head

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_matches_numpy_matmul(orc, dtype):
    s = f32_shape(vocab=2000, top_k=8, hidden=128, dtype=dtype)
    inp = wl.make_inputs_for(s, 21, parts=("h", "W"))
    y, W = inp["h"], inp["W"]
    yd = wl.bf16_bits_to_f32(y).astype(np.float64) if dtype == "bf16" else y.astype(np.float64)
    Wd = wl.bf16_bits_to_f32(W).astype(np.float64) if dtype == "bf16" else W.astype(np.float64)
    out = orc.head(s, y, W, want_logits=True)
    ref = yd @ Wd.T
    np.testing.assert_allclose(out["logits"], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["lse"], logsumexp(ref, axis=1), rtol=1e-13)


def test_head_row_subset(orc):
    s = f32_shape(vocab=700, hidden=64)
    inp = wl.make_inputs_for(s, 22, parts=("h", "W"))
    full = orc.head(s, inp["h"], inp["W"])
    part = orc.head(s, inp["h"], inp["W"], r0=3, nr=2)
    assert np.array_equal(part["ids"], full["ids"][3:5])
    assert np.array_equal(part["logp"], full["logp"][3:5])


def test_logsoftmax_normalises(orc):
    L = np.random.default_rng(23).standard_normal((5, 4000)) * 3
    ids, logp, lse = orc.topk(L, 16)
    np.testing.assert_allclose(np.exp(L - lse[:, None]).sum(1), 1.0, atol=1e-12)
    np.testing.assert_allclose(lse, logsumexp(L, axis=1), rtol=1e-14)
    np.testing.assert_allclose(logp, np.take_along_axis(L, ids, 1) - lse[:, None], atol=1e-14)


def _full_sort_topk(L, K):
    # textbook definition: stable sort by (value desc, id asc)
    out = []
    for row in L:
        order = np.lexsort((np.arange(row.size), -row))
        out.append(order[:K])
    return np.array(out, dtype=np.int32)


def test_topk_matches_full_sort_with_crafted_ties(orc):
    rng = np.random.default_rng(24)
    V = 1537  # ragged
    L = np.round(rng.standard_normal((6, V)) * 4) / 4  # many exact duplicates
    L[0, :] = 0.0
    L[1, ::2] = -0.0
    L[1, 1::2] = 0.0
    L[2, :100] = -np.inf
    L[2, 100:] = -np.inf
    L[2, 1200] = 1.0
    L[2, 5] = 1.0
    L[3, -20:] = 50.0  # maximum in the ragged tail
    L[4, [3, 700, 701, 1536]] = 9.0
    for K in (1, 4, 16, 64):
        ids, _, _ = orc.topk(L, K)
        assert np.array_equal(ids, _full_sort_topk(L, K)), K


def test_topk_all_equal_gives_lowest_ids(orc):
    L = np.full((2, 100), 0.25)
    ids, logp, lse = orc.topk(L, 10)
    assert np.array_equal(ids, np.tile(np.arange(10), (2, 1)))
    np.testing.assert_allclose(lse, 0.25 + math.log(100), atol=1e-15)
    np.testing.assert_allclose(logp, -math.log(100), atol=1e-15)


# --------------------------------------------------------------------------- transitions

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_transitions_match_numpy(orc, dtype):
    s = f32_shape(block=5, vocab=500, top_k=6, rank=32, dtype=dtype)
    inp = wl.make_inputs_for(s, 31, parts=("P", "Q"))
    P, Q = inp["P"], inp["Q"]
    Pd = wl.bf16_bits_to_f32(P).astype(np.float64) if dtype == "bf16" else P.astype(np.float64)
    Qd = wl.bf16_bits_to_f32(Q).astype(np.float64) if dtype == "bf16" else Q.astype(np.float64)
    rng = np.random.default_rng(32)
    ids = rng.integers(0, s.vocab, (s.block, s.top_k)).astype(np.int32)
    anchor = 123
    T = orc.transitions(s, anchor, ids, P, Q)
    np.testing.assert_allclose(T[0, 0], Pd[anchor] @ Qd[ids[1]].T, rtol=1e-13, atol=1e-14)
    assert np.all(T[0, 1:] == 0.0)
    for t in range(2, s.block):
        np.testing.assert_allclose(T[t - 1], Pd[ids[t - 1]] @ Qd[ids[t]].T, rtol=1e-13, atol=1e-14)
    # the predecessor indexes P and the successor indexes Q: swapping the tables changes T
    T_sw = orc.transitions(s, anchor, ids, Q, P)
    assert not np.allclose(T_sw[1], T[1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_transitions_gate(orc, dtype):
    """Context gate H(h_t) of the Inco AI post's pair score
    <A(a) (*) H(h_t), B(b)>: all-ones reproduces the ungated scores exactly;
    a constant c_t in row t scales T_t (and only T_t) by c_t, which pins the
    gate row to the successor's slot; a unit-vector gate e_i keeps the single
    product P[a, i] * Q[b, i]."""
    s = f32_shape(block=5, vocab=400, top_k=5, rank=16, dtype=dtype)
    inp = wl.make_inputs_for(s, 41, parts=("P", "Q"))
    P, Q = inp["P"], inp["Q"]
    Pd = wl.bf16_bits_to_f32(P).astype(np.float64) if dtype == "bf16" else P.astype(np.float64)
    Qd = wl.bf16_bits_to_f32(Q).astype(np.float64) if dtype == "bf16" else Q.astype(np.float64)
    rng = np.random.default_rng(42)
    ids = rng.integers(0, s.vocab, (s.block, s.top_k)).astype(np.int32)
    anchor = 77
    T = orc.transitions(s, anchor, ids, P, Q)
    assert np.array_equal(orc.transitions(s, anchor, ids, P, Q, gate=np.ones((s.block, s.rank))), T)
    c = np.array([100.0, 2.0, 0.5, -3.0, 0.25])  # row 0 (the anchor's slot) is never read
    Tc = orc.transitions(s, anchor, ids, P, Q, gate=np.repeat(c[:, None], s.rank, axis=1))
    for t in range(1, s.block):
        np.testing.assert_allclose(Tc[t - 1], c[t] * T[t - 1], rtol=1e-13, atol=1e-14)
    i = 7
    e = np.zeros((s.block, s.rank))
    e[:, i] = 1.0
    Te = orc.transitions(s, anchor, ids, P, Q, gate=e)
    assert Te[0, 0, 3] == Pd[anchor, i] * Qd[ids[1, 3], i]
    for t in range(2, s.block):
        for j in range(s.top_k):
            for k in range(s.top_k):
                assert Te[t - 1, j, k] == Pd[ids[t - 1, j], i] * Qd[ids[t, k], i]


def test_draft_block_gate_ones_matches_ungated(orc):
    s = wl.shape_of(0)
    inp = wl.make_inputs(0)
    a = orc.draft_block(s, inp["h"], inp["anchor"], inp["wg"], inp["W"], inp["P"], inp["Q"])
    b = orc.draft_block(s, inp["h"], inp["anchor"], inp["wg"], inp["W"], inp["P"], inp["Q"],
                        gate=np.ones((s.rows, s.rank)))
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


# --------------------------------------------------------------------------- walk

def brute_force(logp, T):
    """All K^(B-1) paths; ties go to the reverse-lexicographically smallest
    index sequence (last slot first), which is what lowest-index backpointers
    and the lowest final index produce."""
    B, K = logp.shape
    best = None
    scores = []
    for seq in itertools.product(range(K), repeat=B - 1):
        sc = logp[1, seq[0]] + T[0, 0, seq[0]]
        for t in range(2, B):
            sc += logp[t, seq[t - 1]] + T[t - 1, seq[t - 2], seq[t - 1]]
        scores.append(sc)
        key = (-sc, tuple(reversed(seq)))
        if best is None or key < best[0]:
            best = (key, seq, sc)
    scores.sort(reverse=True)
    second = scores[1] if len(scores) > 1 else -math.inf
    return [-1] + list(best[1]), best[2], scores[0] - second


def random_trellis(rng, B, K, dyadic=False):
    if dyadic:
        logp = rng.integers(-16, 1, (B, K)) / 8.0
        T = rng.integers(-8, 9, (B - 1, K, K)) / 8.0
    else:
        logp = -np.abs(rng.standard_normal((B, K))) * 3
        T = rng.standard_normal((B - 1, K, K)) * 0.5
    T[0, 1:] = 0.0
    logp[0] = 0.0
    return logp, T


@pytest.mark.parametrize("B,K", [(2, 1), (2, 5), (3, 3), (4, 4), (5, 5), (7, 5), (6, 2)])
def test_viterbi_matches_brute_force(orc, B, K):
    rng = np.random.default_rng(100 * B + K)
    for _ in range(5):
        logp, T = random_trellis(rng, B, K)
        idx, score, margin = orc.viterbi(logp, T)
        bidx, bscore, bmargin = brute_force(logp, T)
        assert list(idx) == bidx
        assert abs(score - bscore) < 1e-12
        if math.isinf(bmargin):
            assert math.isinf(margin)
        else:
            assert abs(margin - bmargin) < 1e-12


@pytest.mark.parametrize("B,K", [(3, 4), (4, 4), (5, 3), (7, 4)])
def test_viterbi_exact_ties_dyadic(orc, B, K):
    # dyadic values: every sum is exact, so ties are real ties and the tie rule decides
    rng = np.random.default_rng(7 * B + K)
    ntied = 0
    for _ in range(40):
        logp, T = random_trellis(rng, B, K, dyadic=True)
        idx, score, margin = orc.viterbi(logp, T)
        bidx, bscore, bmargin = brute_force(logp, T)
        assert list(idx) == bidx and score == bscore and margin == bmargin
        ntied += margin == 0.0
    assert ntied > 0  # the cases really exercise the tie rule


def test_viterbi_all_tied_picks_index_zero(orc):
    logp = np.zeros((6, 4))
    T = np.zeros((5, 4, 4))
    idx, score, margin = orc.viterbi(logp, T)
    assert list(idx) == [-1, 0, 0, 0, 0, 0] and score == 0.0 and margin == 0.0


def test_viterbi_zero_transitions_is_per_slot_argmax(orc):
    # DFlash1 behaviour (release-note article: without the selector each slot
    # takes its own argmax): with all pair scores zero the walk reduces to it.
    rng = np.random.default_rng(41)
    logp = -np.abs(rng.standard_normal((8, 16)))
    logp[0] = 0
    T = np.zeros((7, 16, 16))
    idx, score, _ = orc.viterbi(logp, T)
    assert list(idx[1:]) == list(np.argmax(logp[1:], axis=1))
    assert abs(score - logp[1:].max(1).sum()) < 1e-12


def test_viterbi_single_candidate(orc):
    logp = np.array([[0.0], [-1.5], [-0.25], [-2.0]])
    T = np.random.default_rng(42).standard_normal((3, 1, 1))
    idx, score, margin = orc.viterbi(logp, T)
    assert list(idx) == [-1, 0, 0, 0] and math.isinf(margin)
    assert abs(score - (logp[1:, 0].sum() + T.sum())) < 1e-12


def test_viterbi_two_slot_closed_form(orc):
    rng = np.random.default_rng(43)
    logp, T = random_trellis(rng, 2, 9)
    idx, score, _ = orc.viterbi(logp, T)
    v = logp[1] + T[0, 0]
    assert idx[1] == int(np.argmax(v)) and score == v.max()


def test_viterbi_per_slot_shift_invariance(orc):
    rng = np.random.default_rng(44)
    logp, T = random_trellis(rng, 7, 6)
    idx, score, margin = orc.viterbi(logp, T)
    c = rng.standard_normal(7) * 5
    c[0] = 0
    idx2, score2, margin2 = orc.viterbi(logp + c[:, None], T)
    assert list(idx2) == list(idx)
    assert abs(score2 - (score + c[1:].sum())) < 1e-11
    assert abs(margin2 - margin) < 1e-11


def test_figure1_repetition_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "figure1_repetition.json")))
    B, K, r = g["block"], g["top_k"], g["rank"]
    V = 16
    P = np.zeros((V, r), np.float32)
    Q = np.zeros((V, r), np.float32)
    for k, v in g["P"].items():
        P[int(k)] = v
    for k, v in g["Q"].items():
        Q[int(k)] = v
    s = wl.Shape(batch=1, block=B, hidden=16, vocab=V, top_k=K, rank=r, group=16, ksize=2, dtype="f32")
    ids = np.array(g["cand_ids"], np.int32)
    logp = np.array(g["cand_logp"])
    T = orc.transitions(s, g["anchor"], ids, P, Q)
    idx, score, margin = orc.viterbi(logp, T)
    assert list(idx) == g["expected_idx"]
    path = [g["anchor"]] + [int(ids[t, idx[t]]) for t in range(1, B)]
    assert path == g["expected_path"]
    assert score == g["expected_score"] and margin == g["expected_margin"]
    # the independent argmax repeats token 7, which the walk avoids
    assert [g["anchor"]] + [int(ids[t, 0]) for t in range(1, B)] == g["independent_argmax_path"]


# --------------------------------------------------------------------------- end to end

def _numpy_pipeline_paths(s, inp, orc):
    """Independent pipeline from library routines (numpy matmul, logsumexp,
    lexsort) plus brute force over every path; only the conv comes from the
    oracle (it is pinned above)."""
    _, _, yhat = orc.conv(s, inp["h"], inp["wg"])
    y = orc.round_to(s, yhat)
    yd = wl.bf16_bits_to_f32(y).astype(np.float64) if s.dtype == "bf16" else y.astype(np.float64)
    to64 = (lambda a: wl.bf16_bits_to_f32(a).astype(np.float64)) if s.dtype == "bf16" else (lambda a: a.astype(np.float64))
    L = yd @ to64(inp["W"]).T
    lse = logsumexp(L, axis=1)
    ids = _full_sort_topk(L, s.top_k)
    logp = np.take_along_axis(L, ids, 1) - lse[:, None]
    Pd, Qd = to64(inp["P"]), to64(inp["Q"])
    paths, scores = [], []
    for b in range(s.batch):
        rs = slice(b * s.block, (b + 1) * s.block)
        bid, blp = ids[rs], logp[rs]
        T = np.zeros((s.block - 1, s.top_k, s.top_k))
        T[0, 0] = Pd[inp["anchor"][b]] @ Qd[bid[1]].T
        for t in range(2, s.block):
            T[t - 1] = Pd[bid[t - 1]] @ Qd[bid[t]].T
        idx, sc, _ = brute_force(blp, T)
        paths.append([int(inp["anchor"][b])] + [int(bid[t, idx[t]]) for t in range(1, s.block)])
        scores.append(sc)
    return ids, logp, lse, paths, scores


@pytest.mark.parametrize("shape", [
    wl.WORKLOADS[0],
    wl.WORKLOADS[0].with_(batch=3, block=5, vocab=777, top_k=3, dtype="bf16"),
    wl.WORKLOADS[0].with_(batch=2, block=3, hidden=96, group=8, ksize=4, vocab=513, top_k=5),
])
def test_draft_block_matches_independent_pipeline(orc, shape):
    inp = wl.make_inputs_for(shape, 0 if shape == wl.WORKLOADS[0] else 55)
    out = orc.draft_block(shape, inp["h"], inp["anchor"], inp["wg"], inp["W"], inp["P"], inp["Q"])
    ids, logp, lse, paths, scores = _numpy_pipeline_paths(shape, inp, orc)
    assert np.array_equal(out["ids"], ids)
    np.testing.assert_allclose(out["logp"], logp, atol=1e-12)
    np.testing.assert_allclose(out["lse"], lse, rtol=1e-13)
    assert out["path"].tolist() == paths
    np.testing.assert_allclose(out["score"], scores, atol=1e-11)


def test_draft_block_zero_selector_is_dflash1_argmax(orc):
    s = wl.WORKLOADS[0].with_(batch=2)
    inp = wl.make_inputs_for(s, 61)
    zero = np.zeros_like(inp["P"])
    out = orc.draft_block(s, inp["h"], inp["anchor"], inp["wg"], inp["W"], zero, inp["Q"])
    for b in range(s.batch):
        rows = range(b * s.block + 1, (b + 1) * s.block)
        assert out["path"][b, 1:].tolist() == [int(out["ids"][r, 0]) for r in rows]
        assert out["idx"][b, 1:].tolist() == [0] * (s.block - 1)


def test_draft_block_bad_anchor(orc):
    s = wl.WORKLOADS[0].with_(batch=3)
    inp = wl.make_inputs_for(s, 62)
    anchor = inp["anchor"].copy()
    anchor[1] = s.vocab
    anchor[2] = -1
    out = orc.draft_block(s, inp["h"], anchor, inp["wg"], inp["W"], inp["P"], inp["Q"])
    assert out["path"][0, 0] == anchor[0] and np.all(out["path"][0] >= 0)
    assert np.all(out["path"][1:] == -1) and np.all(np.isnan(out["score"][1:]))


# --------------------------------------------------------------------------- other walk rules

def test_greedy_zero_transitions_is_argmax(orc):
    rng = np.random.default_rng(51)
    lp = np.round(rng.standard_normal((6, 5)) * 4) / 4  # dyadic: exact ties happen
    lp[3, 1] = lp[3, 4] = lp[3].max() + 1.0  # a tie for the maximum: the lower index wins
    idx, sc = orc.walk(lp, np.zeros((5, 5, 5)), "greedy")
    want = [int(np.argmax(lp[t])) for t in range(1, 6)]
    assert list(idx) == [-1] + want and want[2] == 1
    assert sc == sum(lp[t, want[t - 1]] for t in range(1, 6))


def test_greedy_one_slot_is_viterbi(orc):
    rng = np.random.default_rng(52)
    lp = rng.standard_normal((2, 7))
    T = rng.standard_normal((1, 7, 7))
    gi, gs = orc.walk(lp, T, "greedy")
    vi, vs, _ = orc.viterbi(lp, T)
    assert list(gi) == list(vi) and gs == vs


def test_greedy_is_myopic(orc):
    """Closed form: the best first step leads into a heavily penalised pair,
    which the best path avoids."""
    lp = np.array([[0.0, 0.0], [0.0, -0.1], [0.0, 0.0]])
    T = np.zeros((2, 2, 2))
    T[1, 0, :] = -5.0
    gi, gs = orc.walk(lp, T, "greedy")
    vi, vs, _ = orc.viterbi(lp, T)
    assert list(gi) == [-1, 0, 0] and gs == -5.0
    assert list(vi) == [-1, 1, 0] and vs == -0.1


def test_sample_uniform_scores_is_floor(orc):
    K = 8
    lp, T = np.zeros((2, K)), np.zeros((1, K, K))
    for i in range(K):
        for frac in (0.0, 0.3, 0.999):
            u = (i + frac) / K
            idx, _ = orc.walk(lp, T, "sample", 1.0, np.array([0.0, u]))
            assert idx[1] == i


def test_sample_tiny_temperature_is_greedy(orc):
    rng = np.random.default_rng(53)
    lp = rng.standard_normal((5, 6))
    T = rng.standard_normal((4, 6, 6))
    gi, gs = orc.walk(lp, T, "greedy")
    for u in (0.0, 0.25, 0.5, 0.9):
        si, ss = orc.walk(lp, T, "sample", 1e-9, np.full(5, u))
        assert list(si) == list(gi) and ss == gs


def test_sample_frequencies_follow_softmax(orc):
    """With N evenly spaced uniforms, candidate k is picked for the uniforms
    in [E_{k-1}, E_k) / E_{K-1}, so its count is N * softmax_k(s / temp) to
    within one."""
    rng = np.random.default_rng(54)
    K, N, temp = 6, 1000, 0.7
    lp = np.vstack([np.zeros(K), rng.standard_normal(K)])
    T = rng.standard_normal((1, K, K))
    s1 = lp[1] + T[0, 0]
    p = np.exp((s1 - s1.max()) / temp)
    p /= p.sum()
    counts = np.zeros(K, int)
    for i in range(N):
        idx, sc = orc.walk(lp, T, "sample", temp, np.array([0.0, (i + 0.5) / N]))
        counts[idx[1]] += 1
        assert sc == s1[idx[1]]
    assert np.all(np.abs(counts - N * p) <= 1.0)
