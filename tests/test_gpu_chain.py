"""GPU parity of chained drafts (mtp_draft_chain_*): step k + 1 takes step k's
draft and block output x.  Every step of every sequence is held to the draft
comparison rules (tests/harness.py, `compare_sequence`) against the oracle's
chain (oracle.draft_chain) on the same seeded inputs.  Where a step is a
genuine near-tie and the two sides pick different (both acceptable) drafts,
the rest of that sequence's chain may differ, so its comparison ends there;
the test reports how many steps were compared.  Also: the chain equals K
separate draft calls fed by hand, bit for bit; an invalid first token
invalidates every step of its sequence only; no-logits mode gives the same
drafts."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import harness

pytestmark = pytest.mark.gpu

INVALID = 0xFFFFFFFF


def _chain_gpu(mtp, dw, fp8, K, tokens, hidden, with_logits=True):
    B, H, V = tokens.size, dw.hidden, dw.vocab
    tk = torch.from_numpy(tokens.astype(np.uint32).view(np.int32)).cuda()
    hd = harness.to_dev_bf16(hidden.reshape(B, H))
    dr = torch.empty((K, B), dtype=torch.int32, device="cuda")
    lg = (torch.empty((K, B, V), dtype=torch.bfloat16, device="cuda") if with_logits else None)
    ws = torch.empty(mtp.mtp_chain_workspace_bytes(H, V, B), dtype=torch.uint8, device="cuda")
    if fp8 is None:
        mtp.mtp_draft_chain_bf16(dw.w, K, B, tk, hd, dr, lg, ws)
    else:
        mtp.mtp_draft_chain_fp8w(dw.w, fp8[0], fp8[1], K, B, tk, hd, dr, lg, ws)
    torch.cuda.synchronize()
    d = dr.cpu().numpy().view(np.uint32)
    return d, (harness.bf16_bits(lg) if lg is not None else None)


def _run(H, V, B, K, seed, bad=None):
    import mtp_draft_head_embed_amd as mtp
    print(f"\n[chain] H={H} V={V} B={B} K={K} seed={seed} bad={bad}", flush=True)
    cfg = synth.custom(H, V, B, seed)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    if bad is not None:
        tokens[bad] = V + 7
    dw = harness.upload(wts)
    qd, sd = harness.quantize_dev(dw)
    qs = oracle.quantize_fp8(wts["lm_head"])
    compared = 0
    for fp8 in (None, (qd, sd)):
        d, lg = _chain_gpu(mtp, dw, fp8, K, tokens, hidden)
        d2, _ = _chain_gpu(mtp, dw, fp8, K, tokens, hidden, with_logits=False)
        assert np.array_equal(d, d2)
        tol = harness.TOL_BF16 if fp8 is None else harness.TOL_FP8
        for b in range(B):
            ref = oracle.draft_chain(wts, int(tokens[b]), hidden[b], K,
                                     None if fp8 is None else qs)
            if ref[0] is None:
                assert np.all(d[:, b] == INVALID), d[:, b]
                continue
            for k in range(K):
                rep = harness.compare_sequence(b, ref[k]["o"], lg[k, b], int(d[k, b]),
                                               ref[k]["draft"], tol)
                assert rep.ok, (k, rep)
                compared += 1
                if int(d[k, b]) != ref[k]["draft"]:
                    print(f"[chain] b={b}: near-tie at step {k} ({rep.gap:.4f}); "
                          "later steps not compared", flush=True)
                    break
        # the chain is K draft calls fed by hand, bit for bit
        tk, hd = tokens.copy(), hidden.copy()
        for k in range(K):
            dk, lk = harness.run_draft(dw, tk, hd, fp8)
            assert np.array_equal(dk, d[k]), k
            assert np.array_equal(lk[tokens < V], lg[k][tokens < V]), k
            xk = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
            ws = mtp.new_workspace(H, V, B)
            mtp.mtp_front(dw.w, B, torch.from_numpy(tk.astype(np.uint32).view(np.int32)).cuda(),
                          harness.to_dev_bf16(hd.reshape(B, H)), xk, ws)
            torch.cuda.synchronize()
            tk, hd = dk.copy(), harness.bf16_bits(xk)
    print(f"[chain] compared {compared} steps", flush=True)
    assert compared >= (B - (bad is not None)) * 2  # most steps are compared


@pytest.mark.parametrize("H,V,B,K,seed", [
    (256, 4096, 1, 4, 3001), (1040, 5003, 3, 3, 3002), (512, 3001, 16, 3, 3003),
])
def test_chain(H, V, B, K, seed):
    _run(H, V, B, K, seed)


def test_chain_invalid_first_token():
    _run(256, 2000, 4, 3, 3004, bad=2)


@pytest.mark.slow
def test_chain_large():
    _run(6144, 154880, 1, 4, 3005)


def test_chain_max_steps():
    """K = 64 (the maximum) chained drafts at a tiny shape."""
    _run(16, 50, 2, 64, 3006)


def test_chain_max_batch():
    _run(64, 700, 64, 2, 3007)
