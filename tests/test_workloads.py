"""The seeded input generators: reproducible bytes, independence from the
thread count and from the tensor's length, the advertised distributions, and
bf16 as the round-to-nearest-even of the fp32 draw.  CPU only."""
import numpy as np
import pytest

import workloads as wl
from workloads import synth


def test_same_seed_same_bytes():
    s = wl.shape_of(0).with_(batch=2, vocab=3001, dtype="bf16")
    a, b = wl.make_inputs_for(s, 5), wl.make_inputs_for(s, 5)
    assert a.keys() == b.keys()
    for k in a:
        assert a[k].dtype == b[k].dtype and np.array_equal(a[k], b[k]), k


def test_seeds_and_tensors_draw_different_streams():
    s = wl.shape_of(0).with_(dtype="f32")
    a, b = wl.make_inputs_for(s, 5), wl.make_inputs_for(s, 6)
    assert not np.array_equal(a["W"], b["W"])
    # P and Q share a shape but not a stream
    assert not np.array_equal(a["P"], a["Q"])


def test_prefix_of_a_longer_tensor():
    """Rows come from per-chunk streams, so a shorter tensor is the prefix of
    a longer one drawn with the same seed (within and across chunks)."""
    short = synth.draw_normal(3, "W", (100, 64), 0.5, "f32")
    long = synth.draw_normal(3, "W", (200, 64), 0.5, "f32")
    assert np.array_equal(short, long[:100])
    a = synth.draw_normal(3, "W", (synth.CHUNK_ROWS + 10, 8), 0.5, "bf16")
    b = synth.draw_normal(3, "W", (2 * synth.CHUNK_ROWS + 5, 8), 0.5, "bf16")
    assert np.array_equal(a, b[: synth.CHUNK_ROWS + 10])


def test_thread_count_does_not_change_bytes(monkeypatch):
    shape = (3 * synth.CHUNK_ROWS + 17, 16)
    many = synth.draw_normal(9, "Q", shape, 1.0, "bf16")
    monkeypatch.setattr(synth, "_threads", lambda: 1)
    one = synth.draw_normal(9, "Q", shape, 1.0, "bf16")
    assert np.array_equal(many, one)


@pytest.mark.parametrize("name,std", [("h", 1.0), ("wg", 1.0 / 16.0), ("W", 3.0 / 16.0), ("P", 0.125)])
def test_advertised_distributions(name, std):
    """h ~ N(0,1), Wg ~ N(0,1/D), W ~ N(0,9/D) at D = 256, P ~ N(0,1/r) at
    r = 64, within a few standard errors (the draw has ~10^6 values)."""
    x = synth.draw_normal(11, name, (4096, 256), std, "f32").astype(np.float64)
    n = x.size
    assert abs(x.mean()) < 5 * std / np.sqrt(n)
    assert abs(x.std() / std - 1.0) < 5 / np.sqrt(2 * n)
    # the tails of a normal: about 4.55 % beyond two standard deviations
    frac = np.mean(np.abs(x) > 2 * std)
    assert abs(frac - 0.0455) < 0.002


def test_bf16_is_rne_of_the_fp32_draw():
    """The bf16 tensor is the fp32 draw rounded to the nearest bf16 value,
    ties to the even pattern, checked against the two neighbouring bf16
    values of each draw in float64."""
    f = synth.draw_normal(21, "h", (64, 512), 1.0, "f32")
    b = synth.draw_normal(21, "h", (64, 512), 1.0, "bf16")
    bits = f.view(np.uint32)
    lo = (bits >> 16).astype(np.uint32)  # truncation toward zero in magnitude
    hi = lo + 1
    to_f64 = lambda p: (p.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = f.astype(np.float64)
    dlo, dhi = np.abs(x - to_f64(lo)), np.abs(x - to_f64(hi))
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi))).astype(np.uint16)
    assert np.array_equal(b, want)


def test_anchor_in_range_and_reproducible():
    a = synth.draw_anchor(4, 1000, 248320)
    assert a.dtype == np.int32 and a.min() >= 0 and a.max() < 248320
    assert np.array_equal(a, synth.draw_anchor(4, 1000, 248320))
    assert len(np.unique(a)) > 990  # 1000 draws from 248 320 values rarely collide
