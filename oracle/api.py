"""numpy wrappers around liboracle.so (test infrastructure only)."""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class _Shape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("batch", "block", "hidden", "vocab", "top_k", "rank", "group", "ksize", "bf16")]


def load():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from .build import build
            build()
        lib = C.CDLL(path)
        P = C.c_void_p
        lib.orc_conv.argtypes = [C.POINTER(_Shape), P, P, P, P, P]
        lib.orc_round.argtypes = [C.POINTER(_Shape), P, P, C.c_int64]
        lib.orc_round.restype = None
        lib.orc_head.argtypes = [C.POINTER(_Shape), P, P, C.c_int, C.c_int, P, P, P, P]
        lib.orc_topk.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P]
        lib.orc_transitions.argtypes = [C.POINTER(_Shape), C.c_int32, P, P, P, P, P]
        lib.orc_viterbi.argtypes = [C.c_int, C.c_int, P, P, P, P, P]
        lib.orc_draft_block.argtypes = [C.POINTER(_Shape)] + [P] * 14
        lib.orc_walk.argtypes = [C.c_int, C.c_int, P, P, C.c_int, C.c_double, P, P, P]
        lib.orc_threads.argtypes = []
        _LIB = lib
    return _LIB


def threads() -> int:
    return int(load().orc_threads())


def _shape(s) -> _Shape:
    return _Shape(s.batch, s.block, s.hidden, s.vocab, s.top_k, s.rank, s.group, s.ksize,
                  1 if s.dtype == "bf16" else 0)


def _tensor(a: np.ndarray, s) -> np.ndarray:
    want = np.uint16 if s.dtype == "bf16" else np.float32
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"expected {want} tensor, got {a.dtype}")
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def conv(s, h, wg):
    """Returns (z, w, yhat) in fp64: tap logits, tap weights, exact conv output."""
    h, wg = _tensor(h, s), _tensor(wg, s)
    Cc = s.groups * s.ksize
    z = np.empty((s.rows, Cc)); w = np.empty((s.rows, Cc)); y = np.empty((s.rows, s.hidden))
    sh = _shape(s)
    if load().orc_conv(C.byref(sh), _p(h), _p(wg), _p(z), _p(w), _p(y)) != 0:
        raise ValueError("orc_conv rejected the shape")
    return z, w, y


def round_to(s, x: np.ndarray) -> np.ndarray:
    """fp64 -> the workload dtype (bf16 bits as uint16, or fp32)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16 if s.dtype == "bf16" else np.float32)
    sh = _shape(s)
    load().orc_round(C.byref(sh), _p(x), _p(out), x.size)
    return out


def head(s, y, W, r0=0, nr=None, want_logits=False):
    """Returns dict(logits?, lse, ids, logp) for rows [r0, r0+nr)."""
    if nr is None:
        nr = s.rows - r0
    y, W = _tensor(y, s), _tensor(W, s)
    logits = np.empty((nr, s.vocab)) if want_logits else None
    lse = np.empty(nr); ids = np.empty((nr, s.top_k), dtype=np.int32); logp = np.empty((nr, s.top_k))
    sh = _shape(s)
    if load().orc_head(C.byref(sh), _p(y), _p(W), r0, nr, _p(logits), _p(lse), _p(ids), _p(logp)) != 0:
        raise ValueError("orc_head failed")
    out = dict(lse=lse, ids=ids, logp=logp)
    if want_logits:
        out["logits"] = logits
    return out


def topk(logits: np.ndarray, K: int):
    """Top-K ids by (logit desc, id asc), log-softmax of those, and lse."""
    L = np.ascontiguousarray(logits, dtype=np.float64)
    nr, V = L.shape
    ids = np.empty((nr, K), dtype=np.int32); logp = np.empty((nr, K)); lse = np.empty(nr)
    if load().orc_topk(nr, V, K, _p(L), _p(ids), _p(logp), _p(lse)) != 0:
        raise ValueError("orc_topk rejected the shape")
    return ids, logp, lse


def _gate(gate, rows, s):
    if gate is None:
        return None
    g = np.ascontiguousarray(gate, dtype=np.float64)
    if g.shape != (rows, s.rank):
        raise ValueError(f"gate must be [{rows}, {s.rank}]")
    return g


def transitions(s, anchor: int, ids_block: np.ndarray, P, Q, gate=None) -> np.ndarray:
    """T [B-1, K, K] for one block; ids_block [B, K] (row 0 ignored); gate
    [B, r] or None (all ones)."""
    ids_block = np.ascontiguousarray(ids_block, dtype=np.int32)
    P, Q = _tensor(P, s), _tensor(Q, s)
    g = _gate(gate, s.block, s)
    T = np.empty((s.block - 1, s.top_k, s.top_k))
    sh = _shape(s)
    if load().orc_transitions(C.byref(sh), int(anchor), _p(ids_block), _p(P), _p(Q), _p(g), _p(T)) != 0:
        raise ValueError("orc_transitions rejected the shape")
    return T


def viterbi(logp_block: np.ndarray, T: np.ndarray):
    """Returns (idx [B] with idx[0] = -1, score, margin) for one block."""
    logp_block = np.ascontiguousarray(logp_block, dtype=np.float64)
    T = np.ascontiguousarray(T, dtype=np.float64)
    B, K = logp_block.shape
    idx = np.empty(B, dtype=np.int32); score = np.empty(1); margin = np.empty(1)
    if load().orc_viterbi(B, K, _p(logp_block), _p(T), _p(idx), _p(score), _p(margin)) != 0:
        raise ValueError("orc_viterbi rejected the shape")
    return idx, float(score[0]), float(margin[0])


def walk(logp_block: np.ndarray, T: np.ndarray, mode: str, temperature: float = 1.0, uniforms=None):
    """Greedy ("greedy") or sampled ("sample") walk of one block: (idx [B]
    with idx[0] = -1, score).  uniforms [B] (entry t for slot t)."""
    logp_block = np.ascontiguousarray(logp_block, dtype=np.float64)
    T = np.ascontiguousarray(T, dtype=np.float64)
    B, K = logp_block.shape
    m = {"greedy": 1, "sample": 2}[mode]
    u = None if uniforms is None else np.ascontiguousarray(uniforms, dtype=np.float64)
    idx = np.empty(B, dtype=np.int32); score = np.empty(1)
    if load().orc_walk(B, K, _p(logp_block), _p(T), m, float(temperature), _p(u), _p(idx), _p(score)) != 0:
        raise ValueError("orc_walk rejected the arguments")
    return idx, float(score[0])


def draft_block(s, h, anchor, wg, W, P, Q, gate=None):
    """End-to-end oracle: dict(path, score, ids, logp, lse, idx, margin);
    gate [rows, r] or None (all ones)."""
    h, wg, W, P, Q = (_tensor(a, s) for a in (h, wg, W, P, Q))
    g = _gate(gate, s.rows, s)
    anchor = np.ascontiguousarray(anchor, dtype=np.int32)
    path = np.empty((s.batch, s.block), dtype=np.int32); score = np.empty(s.batch)
    ids = np.empty((s.rows, s.top_k), dtype=np.int32); logp = np.empty((s.rows, s.top_k))
    lse = np.empty(s.rows); idx = np.empty((s.batch, s.block), dtype=np.int32); margin = np.empty(s.batch)
    sh = _shape(s)
    rc = load().orc_draft_block(C.byref(sh), _p(h), _p(anchor), _p(wg), _p(W), _p(P), _p(Q), _p(g),
                                _p(path), _p(score), _p(ids), _p(logp), _p(lse), _p(idx), _p(margin))
    if rc != 0:
        raise ValueError("orc_draft_block failed")
    return dict(path=path, score=score, ids=ids, logp=logp, lse=lse, idx=idx, margin=margin)
