"""FP8-vs-BF16 draft agreement (the FP8 drafting copy of lm_head may change
which token is proposed, never an emitted token: glm5next_mtp_head.rs,
`head_fp8` field doc).  With random-init weights the share of sequences whose
FP8-head draft equals the BF16-head draft is a synthetic stand-in for how
often the copy would change a proposal, not an acceptance rate.

For the Tiny, Large, Batched and Near-tie configurations, on the same
sequences, the library's agreement rate is set beside the oracle's (the FP8
oracle on the same codes against the BF16 oracle).  Every sequence follows
the comparison rules of tests/harness.py on both heads; wherever both heads'
oracle top-1/top-2 gaps exceed twice their tolerance, both library drafts
equal the oracle's, so the library agrees exactly where the oracle does, and
the two rates can differ only by the share of sequences outside that set.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import harness

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _drafts(dw, tokens, hidden, fp8):
    d, lg = [], []
    for b0 in range(0, tokens.size, 64):  # the ABI takes up to 64 sequences per call
        db, lb = harness.run_draft(dw, tokens[b0:b0 + 64],
                                   np.ascontiguousarray(hidden[b0:b0 + 64]), fp8=fp8)
        d.append(db)
        lg.append(lb)
    return np.concatenate(d), np.concatenate(lg)


def _agreement(name, wts, tokens, hidden):
    dw = harness.upload(wts)
    q, s = harness.quantize_dev(dw)
    ref = oracle.quantize_fp8(wts["lm_head"])
    assert np.array_equal(q.cpu().numpy(), ref[0]) and np.array_equal(s.cpu().numpy(), ref[1])
    g16, l16 = _drafts(dw, tokens, hidden, None)
    g8, l8 = _drafts(dw, tokens, hidden, (q, s))
    n = tokens.size
    o16 = np.zeros(n, np.int64)
    o8 = np.zeros(n, np.int64)
    gated = np.zeros(n, bool)
    for b in range(n):
        r16 = oracle.draft(wts, int(tokens[b]), hidden[b])
        r8 = oracle.draft(wts, int(tokens[b]), hidden[b], fp8=ref)
        p16 = harness.compare_sequence(b, r16["o"], l16[b], int(g16[b]), r16["draft"],
                                       harness.TOL_BF16)
        p8 = harness.compare_sequence(b, r8["o"], l8[b], int(g8[b]), r8["draft"], harness.TOL_FP8)
        assert p16.ok and p8.ok, (name, p16, p8)
        o16[b], o8[b] = r16["draft"], r8["draft"]
        gated[b] = p16.gated_exact and p8.gated_exact
    gpu_agree = g16.astype(np.int64) == g8.astype(np.int64)
    orc_agree = o16 == o8
    assert np.array_equal(gpu_agree[gated], orc_agree[gated]), name
    rate_gpu, rate_orc = gpu_agree.mean(), orc_agree.mean()
    assert abs(rate_gpu - rate_orc) <= (n - gated.sum()) / n + 1e-12
    _say(f"[agreement] {name}: {n} sequences, library {gpu_agree.sum()}/{n} = {rate_gpu:.4f}, "
         f"oracle {orc_agree.sum()}/{n} = {rate_orc:.4f}; both gaps above 2 tol on "
         f"{gated.sum()} (library agrees exactly where the oracle does there)")
    return rate_gpu, rate_orc


def test_agreement_tiny():
    """256 sequences on the Tiny weights (H = 256, V = 4096)."""
    wts = synth.make_weights(synth.CONFIGS["tiny"])
    tokens, hidden = synth.make_inputs(synth.custom(256, 4096, 256, 3001))
    _agreement("tiny", wts, tokens, hidden)


@pytest.mark.slow
def test_agreement_large():
    """32 sequences on the Large weights (H = 6144, V = 154880)."""
    wts = synth.make_weights(synth.CONFIGS["large"])
    tokens, hidden = synth.make_inputs(synth.custom(6144, 154880, 32, 3003))
    _agreement("large", wts, tokens, hidden)


@pytest.mark.slow
def test_agreement_batched():
    """The batched configuration's 16 sequences on its own weights."""
    cfg = synth.CONFIGS["batched"]
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    _agreement("batched", wts, tokens, hidden)


@pytest.mark.slow
def test_agreement_neartie():
    """The near-tie configuration (64 planted ids within 1e-3 of the max per
    sequence): few sequences clear both gates, so the two rates may differ."""
    from tests import neartie
    cfg = synth.CONFIGS["neartie"]
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    nt = neartie.build(cfg, wts, tokens, hidden)
    w2 = dict(wts)
    w2["lm_head"] = nt.lm_head
    _agreement("neartie", w2, tokens, hidden)
