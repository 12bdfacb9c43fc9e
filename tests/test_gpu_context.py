"""GPU parity of the context-row front end (glm5next_mtp_head.rs, `rows_impl`:
row r pairs the embedding of tokens[r + 1] with hiddens[r]) against the
oracle's FP64 rows: each element within the final rounding plus the FP32
summation bound (a plain one-ulp bound fails where the sum nearly cancels),
almost all bit-equal (tests/harness.py, `check_eh_proj_rows`).  Covers the
single-row kernel, the batched split-K sweep (2..16 rows) and the tiled MFMA
GEMM in its tile shapes (128 x 128 with 64-column steps for 17..128 rows,
256 x 256 or 256 x 192 beyond; split over K for few tiles, with ragged row,
column and K tiles)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import harness

pytestmark = pytest.mark.gpu


def _run(H, V, T, seed, bad_row=None, sample=None):
    import mtp_draft_head_embed_amd as mtp
    print(f"\n[context] H={H} V={V} T={T} seed={seed}", flush=True)
    cfg = synth.custom(H, V, T + 1, seed)
    wts = synth.make_weights(cfg)
    tokens, hid = synth.make_inputs(cfg)        # T + 1 tokens and rows; use T rows
    hiddens = np.ascontiguousarray(hid[:T])
    if bad_row is not None:
        tokens[bad_row + 1] = V + 5
    dw = harness.upload(wts)
    tk = torch.from_numpy(tokens.astype(np.uint32).view(np.int32)).cuda()
    hd = harness.to_dev_bf16(hiddens)
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mtp.mtp_context_workspace_bytes(H, T), dtype=torch.uint8, device="cuda")
    mtp.mtp_context_rows(dw.w, T, tk, hd, x, ws)
    torch.cuda.synchronize()
    xg = harness.bf16_bits(x)
    rows = [r for r in (range(T) if sample is None else sample) if r != bad_row]
    # the oracle on the chosen rows only: row r needs tokens[r + 1] and hiddens[r]
    sub_tok = np.concatenate([[0], tokens[np.array(rows) + 1]]).astype(tokens.dtype)
    ref = oracle.context_rows(wts, sub_tok, np.ascontiguousarray(hiddens[rows]))
    st = harness.check_eh_proj_rows(xg[rows], ref["x_unrounded"], ref["concat"],
                                    ref["concat_unrounded"], wts["eh_proj"])
    print(f"[context] {st}", flush=True)
    return xg


@pytest.mark.parametrize("H,V,T,seed", [
    (256, 3000, 1, 80), (256, 3000, 2, 81), (256, 3000, 16, 92), (256, 3000, 17, 93),
    (256, 3000, 37, 82), (256, 3000, 64, 83),
    (256, 3000, 65, 84), (256, 3000, 200, 85), (1040, 2000, 65, 86), (1040, 2000, 130, 87),
    (512, 4000, 300, 88), (1040, 2000, 600, 94), (256, 3000, 255, 95), (256, 3000, 256, 96),
    (1040, 2000, 40, 98), (256, 3000, 128, 97), (256, 3000, 129, 99),
    (2048, 3000, 16, 101),  # 2..16 rows at H a multiple of 1024: the fused front
])
def test_context_rows(H, V, T, seed):
    _run(H, V, T, seed)


def test_context_rows_out_of_range_token():
    """A row whose token is out of range leaves the other rows exact."""
    _run(256, 3000, 100, 89, bad_row=41)
    _run(256, 3000, 10, 90, bad_row=3)
    _run(1024, 3000, 9, 102, bad_row=4)  # the fused front (gather in its prologue)


@pytest.mark.slow
def test_context_rows_large_hidden():
    _run(6144, 20000, 70, 91)


@pytest.mark.slow
def test_context_rows_large_big_tile():
    """H = 6144, T = 600: the 256 x 256 tile with K split four ways; sampled rows
    on both sides of every row-tile edge, checked against the oracle."""
    _run(6144, 20000, 600, 97, sample=[0, 1, 127, 128, 254, 255, 256, 257, 383, 384, 511, 512,
                                       513, 598, 599])


@pytest.mark.slow
def test_context_rows_large_whole_rounds():
    """H = 6144, T = 1024: the 256 x 192 tile on 8 waves (K split two ways, 256
    workgroups, one whole round); sampled rows on both sides of every row-tile
    edge, checked against the oracle."""
    _run(6144, 20000, 1024, 103, sample=[0, 1, 255, 256, 257, 511, 512, 767, 768, 1022, 1023])


def test_context_rows_max_rows():
    """T = 65 536 (the maximum) at H = 16: 256 row tiles of the large tile."""
    _run(16, 100, 65536, 99)


@pytest.mark.slow
def test_context_rows_max_hidden():
    """H = 8192 (the maximum, K = 16 384): sampled rows around the tile edges."""
    _run(8192, 3000, 300, 100, sample=[0, 63, 64, 127, 128, 255, 256, 299])
