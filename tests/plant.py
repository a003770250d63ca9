"""Transition plants of the long-block workload (batch 8, B 16).

For a plant site (b, t, k): u is the anchor (t = 1) or the argmax candidate
of slot t-1 (of the unplanted inputs), v is candidate k of slot t, and
Q[v] <- bf16(Q[v] + 6 * P[u] / |P[u]|^2), computed in fp64 and rounded to
nearest even, which raises the pair score <P[u], Q[v]> by about 6.  Only Q
changes, so the candidates of the unplanted inputs stay the candidates.
Sites that hit the same v are applied in site order.
"""
import numpy as np

import workloads as wl


def plant_pairs(shape, anchor, ids, sites):
    """[(b, t, k, u, v)] for the given sites; ids [rows, K] of the unplanted inputs."""
    out = []
    for b, t, k in sites:
        u = int(anchor[b]) if t == 1 else int(ids[b * shape.block + t - 1, 0])
        v = int(ids[b * shape.block + t, k])
        out.append((b, t, k, u, v))
    return out


def apply_plant(shape, P, Q, pairs):
    """Planted copy of Q (bf16 bit patterns)."""
    import oracle
    Q = Q.copy()
    for _, _, _, u, v in pairs:
        pu = wl.bf16_bits_to_f32(P[u]).astype(np.float64)
        qv = wl.bf16_bits_to_f32(Q[v]).astype(np.float64)
        Q[v] = oracle.round_to(shape, qv + 6.0 * pu / float(pu @ pu))
    return Q
