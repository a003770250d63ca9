"""End-to-end comparison of a GPU draft-block result with the oracle run on
the same seeded inputs (used by the GPU parity and graph-replay tests).

Candidates: ids equal, or every difference swaps entries whose oracle
logits lie within the logit tolerance (a near tie the fp32 logits may order
differently).  Node scores to the relative 2e-3.  Paths: the GPU walks its own
candidates with its own fp32 scores, so the walk is checked on those
candidates with the oracle's fp64 scores of them -- node scores from the
oracle's logits of the GPU's ids minus the oracle's lse, transitions from the
oracle's P.Q.  If every node score moves by at most e (measured: GPU score
minus oracle score) and every transition by at most e_T (the fp32 rounding
bound of a rank-r dot product), every path score moves by at most (B-1)(e +
e_T), so the GPU's best path scores within 2(B-1)(e + e_T) of the oracle's
best on the same candidates.  A block whose oracle margin (best minus second
best) exceeds that bound must take the oracle's path exactly; any other
block must score, under the oracle, within the bound of the best.  No block
is skipped.
"""
from __future__ import annotations

import numpy as np

import workloads as wl
from helpers import as_f64, ids_match_or_explained, rel_err

TOL = 2e-3          # relative (conv, logits, lse, node scores), the stated tolerance
SCORE_TOL = 1e-4    # absolute path-score slack, the stated path tolerance


def dot_bound(s, P, Q, anchor, gids):
    """fp32 rounding bound of the transition dot products of one block:
    r * 2^-24 * max_{a,b} |P[a]| |Q[b]| over its predecessor / successor ids
    (Cauchy-Schwarz bounds sum_i |P[a,i] Q[b,i]|)."""
    pa = np.concatenate([[anchor], gids[1:-1].ravel()])
    pn = np.sqrt((as_f64(s, P[pa]) ** 2).sum(1)).max()
    qn = np.sqrt((as_f64(s, Q[gids[1:].ravel()]) ** 2).sum(1)).max()
    return s.rank * 2.0 ** -24 * pn * qn * 1.01


def check_block_e2e(orc, s, inp, out, blocks=None):
    """out = (path [batch, B], score [batch], ids [rows, K], logp [rows, K])
    from the GPU; inp = the seeded host inputs of shape s.  Compares the
    listed blocks (default: all) with the oracle."""
    path, score, ids, lp = out
    B = s.block
    blocks = list(range(s.batch)) if blocks is None else list(blocks)
    rows = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blocks])
    sub = s.with_(batch=len(blocks))
    h_sub = np.ascontiguousarray(inp["h"][rows])
    ref = orc.draft_block(sub, h_sub, inp["anchor"][blocks], inp["wg"], inp["W"], inp["P"], inp["Q"])
    _, _, yhat = orc.conv(sub, h_sub, inp["wg"])
    y_ref = as_f64(s, orc.round_to(sub, yhat))
    Wd = None

    def ref_row(i):  # oracle logits of a compared row, to explain near-tie reorderings
        nonlocal Wd
        if Wd is None:
            Wd = as_f64(s, inp["W"])
        return Wd @ y_ref[i]

    bad = ids_match_or_explained(ids[rows], ref["ids"], ref_row, tol_abs=TOL * 3.0)
    assert not bad, f"rows with unexplained top-K differences: {bad}"
    ok = np.isfinite(ref["logp"])
    assert rel_err(lp[rows][ok], ref["logp"][ok]) <= TOL
    assert rel_err(score[blocks], ref["score"]) <= TOL
    s1 = s.with_(batch=1)
    n_tight = 0
    for i, b in enumerate(blocks):
        gids = ids[b * B:(b + 1) * B]
        # the oracle's fp64 node scores of the GPU's candidates
        lo = np.zeros((B, s.top_k))
        for t in range(1, B):
            lo[t] = as_f64(s, inp["W"][gids[t]]) @ y_ref[i * B + t] - ref["lse"][i * B + t]
        T = orc.transitions(s1, int(inp["anchor"][b]), gids, inp["P"], inp["Q"])
        idx, best, margin = orc.viterbi(lo, T)
        gidx = [-1] + [int(np.nonzero(gids[t] == path[b, t])[0][0]) for t in range(1, B)]
        e_node = float(np.max(np.abs(lp[b * B + 1:(b + 1) * B].astype(np.float64) - lo[1:])))
        bound = 2 * (B - 1) * (e_node + dot_bound(s, inp["P"], inp["Q"], int(inp["anchor"][b]), gids)) + SCORE_TOL
        assert path[b, 0] == inp["anchor"][b]
        if margin > bound:
            assert gidx == list(idx), f"block {b}: path {gidx} != oracle {list(idx)} (margin {margin:.3g})"
        else:
            n_tight += 1
            g = lo[1, gidx[1]] + T[0, 0, gidx[1]] + sum(lo[t, gidx[t]] + T[t - 1, gidx[t - 1], gidx[t]]
                                                      for t in range(2, B))
            assert abs(g - best) <= bound, f"block {b}: oracle score of the GPU path {g} vs best {best}"
    return n_tight
