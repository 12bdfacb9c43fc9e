"""The near-tie construction itself, checked with the oracle on the CPU at a
reduced size (H = 512, V = 20000, B = 4): planted logits within 1e-3 of c_b,
all rounding to one BF16 value, background at least 0.2 below, the oracle's
draft the lowest planted id, ids disjoint and covering the tile edges."""
import numpy as np

import synth
from tests import neartie


def test_neartie_construction_small():
    cfg = synth.custom(512, 20000, 4, 777, hidden_dist="t3", distinct_tokens=True)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    nt = neartie.build(cfg, wts, tokens, hidden)
    allids = [i for p in nt.planted for i in p]
    assert len(allids) == len(set(allids)) == 4 * neartie.N_PLANT
    assert 0 in nt.planted[0] and cfg.vocab - 1 in nt.planted[1]
    mins = [min(p) for p in nt.planted]
    assert len(set(m // 1024 for m in mins)) == 4  # lowest ids in different regions
    res = neartie.verify(nt, wts, tokens, hidden)
    assert [r["draft"] for r in res] == mins
    # only the planted rows changed
    changed = np.nonzero((nt.lm_head != wts["lm_head"]).any(axis=1))[0]
    assert set(changed.tolist()) <= set(allids)
