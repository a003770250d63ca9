"""Seeded generators for the five workloads of the draft-block path.

Recipe (the same bytes feed the HIP library and the oracle):

* Every tensor is drawn from ``numpy.random.Philox``.  The key of a tensor is
  ``16 * seed + tensor_id`` in its low 64 bits and the index of a 4096-row chunk
  in its high 64 bits, so chunks are independent streams that can be drawn in
  parallel and the bytes do not depend on the thread count.
* Normals are drawn in fp32, multiplied by the fp32 standard deviation and, for
  bf16 workloads, rounded to bf16 with round-to-nearest-even.
* Distributions (hidden size D, selector rank r):
    h ~ N(0, 1); Wg ~ N(0, 1/D); W ~ N(0, 9/D); P, Q ~ N(0, 1/r);
    anchor ~ U[0, V) per block.

Shapes of the workloads follow the isolated-cost setup of the vLLM release
note (page 1, "cost of the added mechanisms": hidden 5120, vocab 248 320,
block 8, K 16) and the checkpoint constants of the RTX 4090 report (page 3,
section 4, ``dflash_config``: block_size 8, conv_group_size 16,
conv_kernel_size 2, selector_rank 256, selector_top_k 16).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

CHUNK_ROWS = 4096

TENSOR_IDS = {"h": 0, "wg": 1, "W": 2, "P": 3, "Q": 4, "anchor": 5, "plant": 6}


@dataclass(frozen=True)
class Shape:
    batch: int
    block: int      # B = 1 + draft slots; slot 0 holds the verified anchor
    hidden: int     # D
    vocab: int      # V
    top_k: int      # K
    rank: int       # r
    group: int      # channels per conv group
    ksize: int      # causal conv taps
    dtype: str      # "f32" or "bf16"

    @property
    def rows(self) -> int:
        return self.batch * self.block

    @property
    def groups(self) -> int:
        return self.hidden // self.group

    def with_(self, **kw) -> "Shape":
        return replace(self, **kw)


WORKLOADS = {
    0: Shape(batch=1, block=4, hidden=64, vocab=1000, top_k=4, rank=16, group=16, ksize=2, dtype="f32"),
    1: Shape(batch=1, block=8, hidden=2560, vocab=151936, top_k=16, rank=256, group=16, ksize=2, dtype="bf16"),
    2: Shape(batch=1, block=8, hidden=5120, vocab=248320, top_k=16, rank=256, group=16, ksize=2, dtype="bf16"),
    3: Shape(batch=32, block=8, hidden=5120, vocab=248320, top_k=16, rank=256, group=16, ksize=2, dtype="bf16"),
    4: Shape(batch=8, block=16, hidden=5120, vocab=248320, top_k=16, rank=256, group=16, ksize=2, dtype="bf16"),
    # selector only: the page shape at batch 1 with the conv off (one tap,
    # so y = h), as the Inco AI post's Table 2 measures path selection
    5: Shape(batch=1, block=8, hidden=5120, vocab=248320, top_k=16, rank=256, group=16, ksize=1, dtype="bf16"),
}


def shape_of(cfg: int) -> Shape:
    return WORKLOADS[cfg]


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the fp32 values they encode (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _philox(seed: int, tensor_id: int, chunk: int) -> np.random.Generator:
    key = (16 * seed + tensor_id) | (chunk << 64)
    return np.random.Generator(np.random.Philox(key=key))


def draw_normal(seed: int, tensor: str, shape: tuple, std: float, dtype: str) -> np.ndarray:
    """N(0, std^2) samples of ``shape``; fp32, or bf16 bit patterns (uint16)."""
    tid = TENSOR_IDS[tensor]
    n_rows = int(shape[0])
    row_len = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1
    out = np.empty((n_rows, row_len), dtype=np.uint16 if dtype == "bf16" else np.float32)
    s32 = np.float32(std)
    n_chunks = (n_rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def work(c: int) -> None:
        r0, r1 = c * CHUNK_ROWS, min(n_rows, (c + 1) * CHUNK_ROWS)
        x = _philox(seed, tid, c).standard_normal((r1 - r0) * row_len, dtype=np.float32)
        x *= s32
        if dtype == "bf16":
            out[r0:r1] = bf16_bits(x).reshape(r1 - r0, row_len)
        else:
            out[r0:r1] = x.reshape(r1 - r0, row_len)

    if n_chunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out.reshape(shape)


def draw_anchor(seed: int, batch: int, vocab: int) -> np.ndarray:
    g = _philox(seed, TENSOR_IDS["anchor"], 0)
    return g.integers(0, vocab, size=batch, dtype=np.int64).astype(np.int32)


def draw_plant_sites(seed: int, batch: int, block: int, top_k: int, fraction: float = 0.10):
    """Random plant sites for the long-block workload: round(fraction * batch
    * (block - 1)) distinct (b, t) pairs with t in 1..block-1, each with a
    candidate index k ~ U[1, top_k - 1] (never the slot's argmax)."""
    g = _philox(seed, TENSOR_IDS["plant"], 0)
    slots = batch * (block - 1)
    n = int(round(fraction * slots))
    pick = np.sort(g.choice(slots, size=n, replace=False))
    ks = g.integers(1, top_k, size=n)
    return [(int(i // (block - 1)), int(i % (block - 1)) + 1, int(k)) for i, k in zip(pick, ks)]


def make_inputs_for(shape: Shape, seed: int, parts=("h", "wg", "W", "P", "Q", "anchor")) -> dict:
    """Draw the inputs of one workload.

    Returns numpy arrays: ``h [rows, D]``, ``wg [D, G*ks]`` (the generator
    weight in its mathematical layout: column ``g*ks + j`` gives tap ``j`` of
    group ``g``), ``W [V, D]``, ``P [V, r]``, ``Q [V, r]`` (fp32, or bf16 bit
    patterns as uint16) and ``anchor [batch]`` int32.
    """
    s = shape
    D = s.hidden
    out = {}
    if "h" in parts:
        out["h"] = draw_normal(seed, "h", (s.rows, D), 1.0, s.dtype)
    if "wg" in parts:
        out["wg"] = draw_normal(seed, "wg", (D, s.groups * s.ksize), float(np.sqrt(1.0 / D)), s.dtype)
    if "W" in parts:
        out["W"] = draw_normal(seed, "W", (s.vocab, D), float(np.sqrt(9.0 / D)), s.dtype)
    if "P" in parts:
        out["P"] = draw_normal(seed, "P", (s.vocab, s.rank), float(np.sqrt(1.0 / s.rank)), s.dtype)
    if "Q" in parts:
        out["Q"] = draw_normal(seed, "Q", (s.vocab, s.rank), float(np.sqrt(1.0 / s.rank)), s.dtype)
    if "anchor" in parts:
        out["anchor"] = draw_anchor(seed, s.batch, s.vocab)
    return out


def make_inputs(cfg: int, parts=("h", "wg", "W", "P", "Q", "anchor")) -> dict:
    """Inputs of workload ``cfg`` (0..4) with its own seed (= cfg).

    Workload 4 additionally plants transition bonuses; that step needs the
    oracle's candidates and lives with the tests, not here.
    """
    return make_inputs_for(WORKLOADS[cfg], cfg, parts)
