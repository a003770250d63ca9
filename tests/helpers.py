"""Shared test helpers: device transfer, the comparison metric, and the
comparison of a GPU run against the oracle."""
from __future__ import annotations

import numpy as np

import workloads as wl


def rel_err(x, r) -> float:
    """max_i |x_i - r_i| / max(|r_i|, rms(r)): relative error for ordinary
    entries, scaled by the rms of the reference near zero."""
    x = np.asarray(x, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r))) or 1.0
    return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), rms)))


def to_dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def from_dev(t) -> np.ndarray:
    import torch
    a = t.detach().cpu()
    if a.dtype == torch.int16:
        return a.numpy().view(np.uint16)
    return a.numpy()


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda")


def as_f64(s: wl.Shape, a: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(a).astype(np.float64) if s.dtype == "bf16" else np.asarray(a, np.float64)


def wg_channel_major(wg: np.ndarray) -> np.ndarray:
    """[D, G*ks] generator -> the library's channel-major [G*ks, D] layout."""
    return np.ascontiguousarray(wg.T)


def ids_match_or_explained(gpu_ids, ref_ids, ref_logits_row_fn, tol_abs):
    """True if top-K id lists agree, or every disagreement swaps entries whose
    reference logits are within tol_abs (a near tie the fp32 GPU logits may
    order differently)."""
    gpu_ids = np.asarray(gpu_ids)
    ref_ids = np.asarray(ref_ids)
    bad = []
    for i in range(gpu_ids.shape[0]):
        if np.array_equal(gpu_ids[i], ref_ids[i]):
            continue
        L = ref_logits_row_fn(i)
        g = np.sort(L[gpu_ids[i]])[::-1]
        r = np.sort(L[ref_ids[i]])[::-1]
        if np.max(np.abs(g - r)) > tol_abs:
            bad.append(i)
    return bad


def topk_of(logits, K):
    """Direct check of a top-K result against the logits it was taken from:
    the K largest entries of each row (larger first, equal values by smaller
    id, -0 equal to +0) and the row's log-sum-exp in fp64.  A property of the
    returned logits, not a second implementation of the method."""
    L = np.asarray(logits, np.float32)
    rows, V = L.shape
    kth = np.partition(L, V - K, axis=1)[:, V - K]
    ids = np.empty((rows, K), np.int32)
    for i in range(rows):
        cand = np.nonzero(L[i] >= kth[i])[0]
        order = np.lexsort((cand, -L[i, cand].astype(np.float64)))
        ids[i] = cand[order[:K]]
    Ld = L.astype(np.float64)
    m = Ld.max(axis=1)
    lse = m + np.log(np.exp(Ld - m[:, None]).sum(axis=1))
    return ids, lse
