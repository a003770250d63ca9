"""Writes plant_w4.json: the oracle's reference for the long-block workload
(batch 8, B 16, D 5120, V 248320, K 16, r 256) with transition plants.

Run from the repository root: python tests/golden/make_plant_w4.py
It calls only the seeded generators and the oracle (about a minute on 8
cores).
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from plant import apply_plant, plant_pairs  # noqa: E402


def compute():
    """The fixture's content, from the seeded generators and the oracle."""
    s = wl.shape_of(4)
    t0 = time.time()
    inp = wl.make_inputs(4)
    print(f"inputs {time.time() - t0:.1f} s", flush=True)
    _, _, yhat = oracle.conv(s, inp["h"], inp["wg"])
    y = oracle.round_to(s, yhat)
    t0 = time.time()
    hd = oracle.head(s, y, inp["W"])
    print(f"oracle head {time.time() - t0:.1f} s", flush=True)
    sites = wl.draw_plant_sites(4, s.batch, s.block, s.top_k)
    pairs = plant_pairs(s, inp["anchor"], hd["ids"], sites)
    Qp = apply_plant(s, inp["P"], inp["Q"], pairs)
    res = oracle.draft_block(s, inp["h"], inp["anchor"], inp["wg"], inp["W"], inp["P"], Qp)
    assert np.array_equal(res["ids"], hd["ids"])  # the plant leaves the candidates unchanged
    argmax_paths = [[int(inp["anchor"][b])] + [int(hd["ids"][b * s.block + t, 0]) for t in range(1, s.block)]
                    for b in range(s.batch)]
    # a planted site deviates if the walk does not take the slot's argmax there
    deviating = [(b, t) for b, t, *_ in pairs if res["idx"][b, t] != 0]
    out = {
        "workload": "batch 8, B 16, D 5120, V 248320, K 16, r 256, bf16; seed 4; plants on 10% of draft slots",
        "generator": "workloads.make_inputs(4), sites workloads.draw_plant_sites(4, 8, 16, 16), tests/plant.py",
        "sites": [list(p) for p in pairs],
        "cand_ids": hd["ids"].tolist(),
        "lse": hd["lse"].tolist(),
        "path": res["path"].tolist(),
        "idx": res["idx"].tolist(),
        "score": res["score"].tolist(),
        "margin": res["margin"].tolist(),
        "argmax_path": argmax_paths,
        "n_sites": len(pairs),
        "n_sites_deviating": len(deviating),
        "n_blocks_off_argmax": int(sum(res["path"][b].tolist() != argmax_paths[b] for b in range(s.batch))),
    }
    return out


def main():
    out = compute()
    s = wl.shape_of(4)
    path = os.path.join(ROOT, "tests", "golden", "plant_w4.json")
    json.dump(out, open(path, "w"))
    print(f"{out['n_sites']} sites, {out['n_sites_deviating']} deviate from the argmax; "
          f"{out['n_blocks_off_argmax']} of {s.batch} block paths differ from the per-slot argmax")


if __name__ == "__main__":
    main()
