"""The allocation-free draft call (mtp_draft_static) against the workspace
calls it stands in for (mtp_draft_bf16, mtp_draft_fp8w), through the C ABI:
the same kernels on the same inputs, so drafts and logits must be equal bit
for bit.  Two calls in a row per head, the second with a smaller input (fewer
sequences, and the single-sequence kernels), so the second call runs on scratch
that still holds the first call's contents."""
import numpy as np
import pytest
import torch

import synth
from tests import harness

pytestmark = pytest.mark.gpu


def _call_static(dw, tokens, hidden, fp8):
    import mtp_draft_head_embed_amd as mtp
    B = int(tokens.size)
    tk = torch.from_numpy(tokens.astype(np.uint32).view(np.int32)).cuda()
    hd = harness.to_dev_bf16(hidden.reshape(B, dw.hidden))
    dr = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    lg = torch.zeros((B, dw.vocab), dtype=torch.bfloat16, device="cuda")
    q, s = fp8 if fp8 is not None else (None, None)
    mtp.mtp_draft_static(dw.w, q, s, B, tk, hd, dr, lg)
    torch.cuda.synchronize()
    return dr.cpu().numpy().view(np.uint32), harness.bf16_bits(lg)


@pytest.mark.parametrize("H,V", [(1024, 20011), (6144, 9001)])
def test_static_matches_workspace_calls(H, V):
    print(f"\n[no-alloc] H={H} V={V}", flush=True)
    cfg = synth.custom(H, V, 32, 5000 + H)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    tokens[3] = V + 1  # an invalid token in the first call
    dw = harness.upload(wts)
    q, s = harness.quantize_dev(dw)
    for fp8 in (None, (q, s)):
        for B in (32, 1):  # the second call smaller, on the single-sequence kernels
            tk, hd = tokens[:B].copy(), np.ascontiguousarray(hidden[:B])
            d_s, l_s = _call_static(dw, tk, hd, fp8)
            d_w, l_w = harness.run_draft(dw, tk, hd, fp8=fp8)
            assert np.array_equal(d_s, d_w), (fp8 is not None, B)
            assert np.array_equal(l_s, l_w), (fp8 is not None, B)
        # and again a batched call after the single one (scratch reused across layouts)
        tk, hd = tokens[:5].copy(), np.ascontiguousarray(hidden[:5])
        d_s, l_s = _call_static(dw, tk, hd, fp8)
        d_w, l_w = harness.run_draft(dw, tk, hd, fp8=fp8)
        assert np.array_equal(d_s, d_w) and np.array_equal(l_s, l_w)
    assert d_s.size == 5


def test_static_rejects_oversized_shape():
    import mtp_draft_head_embed_amd as mtp
    H, V, B = 8192, 1000, 64
    cfg = synth.custom(H, V, B, 5100)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    dw = harness.upload(wts)
    tk = torch.from_numpy(tokens.view(np.int32)).cuda()
    hd = harness.to_dev_bf16(hidden)
    dr = torch.empty(B, dtype=torch.int32, device="cuda")
    with pytest.raises(mtp.MtpError) as ei:
        mtp.mtp_draft_static(dw.w, None, None, B, tk, hd, dr, None)
    assert ei.value.status == mtp.MTP_ERR_SCRATCH
