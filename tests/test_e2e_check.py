"""CPU checks of the end-to-end comparison itself (tests/e2e_check.py): it
accepts the oracle's own result rounded to the GPU's output types, and it
rejects a wrong path, a wrong candidate and a wrong score."""
import numpy as np
import pytest

import workloads as wl
import e2e_check as e2e


def S(**kw):
    base = dict(batch=3, block=6, hidden=64, vocab=700, top_k=8, rank=32, group=16, ksize=2, dtype="bf16")
    base.update(kw)
    return wl.Shape(**base)


def oracle_as_gpu(orc, s, inp):
    ref = orc.draft_block(s, inp["h"], inp["anchor"], inp["wg"], inp["W"], inp["P"], inp["Q"])
    return [ref["path"].astype(np.int32), ref["score"].astype(np.float32), ref["ids"].astype(np.int32),
            ref["logp"].astype(np.float32)], ref


@pytest.mark.parametrize("s", [S(), S(dtype="f32", ksize=4, group=8), S(batch=2, block=3, top_k=1)], ids=str)
def test_accepts_the_oracle_result(orc, s):
    inp = wl.make_inputs_for(s, 5)
    out, _ = oracle_as_gpu(orc, s, inp)
    e2e.check_block_e2e(orc, s, inp, out)


def test_rejects_planted_mistakes(orc):
    s = S()
    inp = wl.make_inputs_for(s, 6)
    out, ref = oracle_as_gpu(orc, s, inp)
    b = int(np.argmax(ref["margin"]))  # a block whose best path is clear
    # another path through the same candidates
    bad = [x.copy() for x in out]
    t = s.block - 1
    k = (ref["idx"][b, t] + 1) % s.top_k
    bad[0][b, t] = out[2][b * s.block + t, k]
    with pytest.raises(AssertionError):
        e2e.check_block_e2e(orc, s, inp, bad)
    # a candidate list with a token that is far from the top K
    bad = [x.copy() for x in out]
    row = b * s.block + 2
    far = [v for v in range(s.vocab) if v not in set(out[2][row].tolist())][0]
    bad[2][row, -1] = far
    with pytest.raises(AssertionError):
        e2e.check_block_e2e(orc, s, inp, bad)
    # a path score off by more than the tolerance
    bad = [x.copy() for x in out]
    bad[1][b] += 0.1 * max(1.0, abs(float(bad[1][b])))
    with pytest.raises(AssertionError):
        e2e.check_block_e2e(orc, s, inp, bad)
