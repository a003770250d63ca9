"""CPU checks of the long-block plant fixture (tests/golden/plant_w4.json)."""
import json
import os

import pytest

import workloads as wl

G = os.path.join(os.path.dirname(__file__), "golden", "plant_w4.json")


def test_plant_sites_are_the_seeded_draw():
    g = json.load(open(G))
    s = wl.shape_of(4)
    sites = wl.draw_plant_sites(4, s.batch, s.block, s.top_k)
    assert len(sites) == round(0.10 * s.batch * (s.block - 1)) == g["n_sites"] == 12
    assert [tuple(x[:3]) for x in g["sites"]] == sites
    for b, t, k, u, v in g["sites"]:
        assert 0 <= b < s.batch and 1 <= t < s.block and 1 <= k < s.top_k
        assert 0 <= u < s.vocab and 0 <= v < s.vocab
        assert g["cand_ids"][b * s.block + t][k] == v
        assert u == (g["path"][b][0] if t == 1 else g["cand_ids"][b * s.block + t - 1][0])


def test_plants_move_the_oracle_walk():
    g = json.load(open(G))
    # most plants pull the walk off the per-slot argmax (a node-logit plant
    # alone could not: node scores enter both rules identically)
    assert g["n_sites_deviating"] >= g["n_sites"] // 2
    assert g["n_blocks_off_argmax"] >= 1
    for b, path in enumerate(g["path"]):
        assert path[0] == g["argmax_path"][b][0]


@pytest.mark.slow
def test_fixture_recomputes_from_the_oracle():
    """The stored fixture equals what the oracle computes now from the seeded
    inputs (candidates, lse, paths, indices, scores, margins and counts), so
    a change to the oracle or the generators cannot leave it stale.  About a
    minute on 8 cores."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_plant_w4", os.path.join(os.path.dirname(__file__), "golden", "make_plant_w4.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    fresh = json.loads(json.dumps(mod.compute()))
    stored = json.load(open(G))
    assert fresh.keys() == stored.keys()
    for k in stored:
        assert fresh[k] == stored[k], k
