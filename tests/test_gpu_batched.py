"""GPU parity of the batched (B >= 2) sweep in every matrix-core kernel
variant the launcher picks, against the FP64 oracle.

The batched head streams lm_head once for all B sequences; which kernel runs
depends on B and H only:
  * 2 <= B <= 16 at H <= 6144: the tile kernel (tile_gemm.hip), one 16-row
    tile per workgroup with K split over its 8 waves; the wave's slice of each
    row is 2, 4 or 6 segments of 128 bytes per chunk, one chunk (FP8, and BF16
    to H = 3072) or two (BF16 above);
  * otherwise batch tiles of 16 sequences: one (B <= 16), two (17-32), three
    (33-48) or four (49-64), each with its own accumulators, K-chunked
    ("multi-chunk") when B staged activation rows of H columns do not fit in
    LDS: at H = 6144 from B = 17 (two tiles), at H = 8192 from B = 9;
  * K-chunked split-K eh_proj: at H = 6144 from B = 50, at H = 8192 from B = 28;
  * 2 <= B <= 16 at H a multiple of 1024 up to 6144: eh_proj in the tile
    kernel with the gather and both norms in its prologue (K split in four,
    H / 1024 segments per wave slice); other shapes write the concat rows
    first and run the split-K MFMA eh_proj.
V = 20 011 keeps the oracle cheap (the choice of kernel does not depend on V)
and leaves a ragged last row tile.

Per case: FP8 codes bit-exact; for every sequence the draft is the lowest
index of its own largest logit; for sampled sequences (all when B <= 17, else
the first and last of every batch tile and their neighbours) every logit of
both heads against the oracle under the comparison rules of tests/harness.py,
and the block input x of `mtp_front` (the same batched front half) against the
oracle's unrounded x (tests/harness.py, `check_eh_proj_rows`).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import harness

pytestmark = pytest.mark.gpu

V_CASE = 20011

CASES = [
    # (H, B, seed, what the launcher runs)
    (6144, 12, 201, "tile kernel, 6-segment chunks (BF16 two per tile)"),
    (6144, 16, 202, "tile kernel at the batched configuration's B"),
    (4096, 6, 212, "tile kernel, 4-segment chunks (BF16 two per tile)"),
    (3088, 2, 213, "tile kernel, ragged last slice (BF16 7 of 8 segments); concat-first front"),
    (1024, 3, 214, "fused front, 1 segment per slice"),
    (2048, 7, 215, "fused front, 2 segments per slice"),
    (3072, 16, 216, "fused front, 3 segments per slice"),
    (5120, 11, 217, "fused front, 5 segments per slice"),
    (6144, 17, 203, "K-chunked head, two batch tiles"),
    (6144, 33, 204, "K-chunked head, three batch tiles"),
    (6144, 50, 205, "K-chunked head, four tiles; first K-chunked split-K eh_proj"),
    (6144, 64, 206, "K-chunked head, four tiles; K-chunked eh_proj (largest batch)"),
    (8192, 9, 207, "K-chunked one-tile head from B = 9 at the largest hidden"),
    (8192, 28, 208, "K-chunked head, two tiles; K-chunked eh_proj at the largest hidden"),
    (2048, 17, 209, "single-chunk head, two batch tiles"),
    (1024, 48, 210, "single-chunk head, three batch tiles"),
    (1024, 56, 211, "single-chunk head, four batch tiles"),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def sample_sequences(B: int) -> list:
    if B <= 17:
        return list(range(B))
    s = {0, 1, B - 2, B - 1}
    for t in range(0, B, 16):
        s.update({t - 1, t, t + 1, t + 15})
    return sorted(b for b in s if 0 <= b < B)


def _self_consistent(d, lg):
    g = harness.bits_to_f64(lg)
    for b in range(d.size):
        own = int(np.nonzero(g[b] == g[b].max())[0][0])
        assert int(d[b]) == own, (b, int(d[b]), own)


@pytest.mark.slow
@pytest.mark.parametrize("H,B,seed,what", CASES, ids=[f"H{c[0]}-B{c[1]}" for c in CASES])
def test_batched_variant(H, B, seed, what):
    import mtp_draft_head_embed_amd as mtp
    _say(f"\n[batched] H={H} V={V_CASE} B={B} seed={seed}: {what}")
    cfg = synth.custom(H, V_CASE, B, seed, distinct_tokens=True)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    dw = harness.upload(wts)
    q, s = harness.quantize_dev(dw)
    ref = oracle.quantize_fp8(wts["lm_head"])
    assert np.array_equal(q.cpu().numpy(), ref[0])
    assert np.array_equal(s.cpu().numpy(), ref[1])
    d16, lg16 = harness.run_draft(dw, tokens, hidden)
    d8, lg8 = harness.run_draft(dw, tokens, hidden, fp8=(q, s))
    _self_consistent(d16, lg16)
    _self_consistent(d8, lg8)

    # the block input x from the same batched front half
    tk = torch.from_numpy(tokens.astype(np.uint32).view(np.int32)).cuda()
    x = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
    ws = mtp.new_workspace(H, V_CASE, B)
    mtp.mtp_front(dw.w, B, tk, harness.to_dev_bf16(hidden), x, ws)
    torch.cuda.synchronize()
    xg = harness.bf16_bits(x)

    picks = sample_sequences(B)
    xs, xu, cc, cu = [], [], [], []
    worst = {"bf16": 0.0, "fp8": 0.0}
    for b in picks:
        for path, d, lg, fp8 in (("bf16", d16, lg16, None), ("fp8", d8, lg8, ref)):
            r = oracle.draft(wts, int(tokens[b]), hidden[b], fp8=fp8)
            rep = harness.compare_sequence(b, r["o"], lg[b], int(d[b]), r["draft"],
                                           harness.TOL_FP8 if fp8 is not None else harness.TOL_BF16)
            assert rep.ok, (path, rep)
            worst[path] = max(worst[path], rep.max_err / rep.tol)
            if fp8 is None:
                xs.append(xg[b])
                xu.append(r["x_unrounded"])
                cc.append(r["concat"])
                cu.append(r["concat_unrounded"])
    st = harness.check_eh_proj_rows(np.stack(xs), np.stack(xu), np.stack(cc), np.stack(cu),
                                    wts["eh_proj"])
    _say(f"[batched] H={H} B={B}: {len(picks)} sequences against the oracle, worst logit error "
         f"{worst['bf16']:.3f} tol (BF16) / {worst['fp8']:.3f} tol (FP8); x: {st}")


@pytest.mark.parametrize("V,B,seed", [(300, 4, 221), (4099, 9, 222), (20, 16, 223)])
def test_tile_head_small_vocab(V, B, seed):
    """Vocabularies with fewer 16-row tiles than two grid rounds: the grid is one
    workgroup per tile (V = 300: 19 of them, so fewer than eight tile pools, and
    every pool empty), one per CU with the second round partly empty
    (V = 4 099: 257 tiles, the last holding 3 rows), or fewer tiles than
    sequences (V = 20: 2 tiles, B = 16; two workgroups).  Every logit of every
    sequence, both heads, against the oracle."""
    _say(f"\n[batched] small vocabulary H=1024 V={V} B={B} seed={seed}")
    cfg = synth.custom(1024, V, B, seed, distinct_tokens=True)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    dw = harness.upload(wts)
    q, s = harness.quantize_dev(dw)
    ref = oracle.quantize_fp8(wts["lm_head"])
    d16, lg16 = harness.run_draft(dw, tokens, hidden)
    d8, lg8 = harness.run_draft(dw, tokens, hidden, fp8=(q, s))
    _self_consistent(d16, lg16)
    _self_consistent(d8, lg8)
    for b in range(B):
        for d, lg, fp8 in ((d16, lg16, None), (d8, lg8, ref)):
            r = oracle.draft(wts, int(tokens[b]), hidden[b], fp8=fp8)
            rep = harness.compare_sequence(b, r["o"], lg[b], int(d[b]), r["draft"],
                                           harness.TOL_FP8 if fp8 is not None else harness.TOL_BF16)
            assert rep.ok, (fp8 is not None, rep)
