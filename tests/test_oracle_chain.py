"""Pins of the oracle's chained drafts (oracle.draft_chain) in closed form.

With unit norm weights, lm_head = I (V = H) and eh_proj built from the cyclic
shift P (P v)_i = v_{i-1}, every draft is an argmax moved one place:
  * eh_proj = [P | 0]: x = P enorm(embed[token]), so draft = token + 1 when
    embed row t peaks at t; a chain that feeds back its draft as the next token
    counts t + 1, t + 2, ... (a chain that kept the first token would repeat);
  * eh_proj = [0 | P]: x = P hnorm(hidden), so draft = argmax(hidden) + 1; a
    chain that feeds back x as the next hidden counts a + 1, a + 2, ... (one
    that kept the first hidden would repeat a + 1).
"""
import numpy as np
import pytest

import oracle
from synth import to_bf16


def bf16_bits(a):
    return to_bf16(np.asarray(a, dtype=np.float32))

H = 16


def _weights(block: str, embed=None):
    one = np.full(H, 1.0)
    P = np.zeros((H, H))
    for i in range(H):
        P[i, (i - 1) % H] = 1.0
    Z = np.zeros((H, H))
    eh = np.hstack([P, Z]) if block == "token" else np.hstack([Z, P])
    if embed is None:
        embed = np.full((H, H), 0.25) + 3.0 * np.eye(H)   # row t peaks at t
    return {
        "embed": bf16_bits(embed), "enorm_w": bf16_bits(one), "hnorm_w": bf16_bits(one),
        "head_norm_w": bf16_bits(one), "eh_proj": bf16_bits(eh), "lm_head": bf16_bits(np.eye(H)),
        "rms_eps": 1e-6,
    }


@pytest.mark.parametrize("t0", [0, 5, 15])
def test_token_fed_back(t0):
    w = _weights("token")
    hidden = bf16_bits(np.linspace(-1.0, 1.0, H))
    res = oracle.draft_chain(w, t0, hidden, 6)
    assert [r["draft"] for r in res] == [(t0 + k) % H for k in range(1, 7)]


@pytest.mark.parametrize("a", [0, 7, 15])
def test_hidden_fed_back(a):
    w = _weights("hidden")
    h = np.full(H, 0.5)
    h[a] = 4.0
    res = oracle.draft_chain(w, 3, bf16_bits(h), 5)
    assert [r["draft"] for r in res] == [(a + k) % H for k in range(1, 6)]
    # each step's x is the previous x (normalised) moved one place
    for k in range(1, 5):
        assert np.array_equal(np.argsort(-oracle.bf16_to_f64(res[k]["x"]), kind="stable")[0],
                              (a + k + 1) % H)


def test_single_step_is_one_draft_and_invalid_token_ends():
    w = _weights("token")
    hidden = bf16_bits(np.linspace(-1.0, 1.0, H))
    one = oracle.draft(w, 4, hidden)
    ch = oracle.draft_chain(w, 4, hidden, 1)
    assert len(ch) == 1 and ch[0]["draft"] == one["draft"]
    assert np.array_equal(ch[0]["logits"], one["logits"])
    assert oracle.draft_chain(w, H + 3, hidden, 4) == [None]


def test_block_output_not_normed_output_fed_back():
    """head_norm_w = 0.5 at index 4 only: hidden peaks 4.0 at 3 and 3.5 at 9
    give x_1 peaks at 4 and 10; the head norm halves the one at 4, so draft 1
    is 10.  Fed back x_1 keeps the 4.0 peak, so draft 2 is 5 (then 6, 7);
    feeding back the normed xn_1 instead would give 11."""
    w = _weights("hidden")
    hw = np.full(H, 1.0)
    hw[4] = 0.5
    w["head_norm_w"] = bf16_bits(hw)
    h = np.full(H, 0.5)
    h[3], h[9] = 4.0, 3.5
    res = oracle.draft_chain(w, 2, bf16_bits(h), 4)
    assert [r["draft"] for r in res] == [10, 5, 6, 7]
