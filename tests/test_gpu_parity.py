"""GPU parity: the HIP path through the C ABI against the FP64 oracle.

Comparison rules (tests/harness.py): FP8 bytes and scales bit-exact; logits
within 2e-2 sigma (BF16 head) / 6e-2 sigma (FP8 head, against the FP8 oracle);
drafts exact wherever the oracle's top-1/top-2 gap exceeds twice the
tolerance, always the lowest index of the GPU's own largest logit, and always in
the oracle's near-max set.

Shapes: small ones the oracle finishes in seconds (several row tiles, ragged
column chunks and a ragged vocab), the edge shapes (H = 16, V = 1, H = 8192,
B = 64), and the full configurations (Mid, Large, Batched) in the launch
configuration the benchmark times.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import harness

pytestmark = pytest.mark.gpu

SMALL = [
    # (hidden, vocab, batch, seed)
    (256, 4096, 1, 1001),     # the Tiny configuration's shape
    (1040, 5003, 3, 31),      # ragged column chunk (2 x 512 + 16) and ragged vocab
    (16, 1, 1, 32),           # smallest hidden, a one-token vocabulary
    (16, 7, 2, 33),
    (8192, 2049, 2, 34),      # largest hidden
    (512, 700, 64, 35),       # largest batch
    (2064, 1999, 5, 36),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check_all(cfg, wts, tokens, hidden, dw, fp8_dev=None, fp8_ref=None, with_logits=True):
    d, lg = harness.run_draft(dw, tokens, hidden, fp8=fp8_dev, with_logits=with_logits)
    reps = []
    for b in range(tokens.size):
        r = oracle.draft(wts, int(tokens[b]), hidden[b], fp8=fp8_ref)
        rep = harness.compare_sequence(b, r["o"], None if lg is None else lg[b], int(d[b]),
                                       r["draft"],
                                       harness.TOL_FP8 if fp8_ref is not None else harness.TOL_BF16)
        reps.append(rep)
        assert rep.ok, (cfg, rep)
    return d, lg, reps


@pytest.mark.parametrize("H,V,B,seed", SMALL)
def test_small_shapes_bf16_and_fp8(H, V, B, seed):
    _say(f"\n[parity] H={H} V={V} B={B} seed={seed}")
    cfg = synth.custom(H, V, B, seed)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    dw = harness.upload(wts)
    _check_all(cfg, wts, tokens, hidden, dw)
    q, s = harness.quantize_dev(dw)
    ref = oracle.quantize_fp8(wts["lm_head"])
    assert np.array_equal(q.cpu().numpy(), ref[0])
    assert np.array_equal(s.cpu().numpy(), ref[1])
    _check_all(cfg, wts, tokens, hidden, dw, (q, s), ref)


def test_quantiser_exhaustive_rows():
    """Rows [448, w, 0...] for every finite BF16 |w| <= 448 (scale exactly 1)
    and rows [w, 0...] for every finite nonzero BF16 w (the scale path), plus
    all-zero and signed-zero rows: GPU codes and scales bit-exact."""
    _say("\n[quantiser] exhaustive BF16 rows")
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    fin = np.isfinite(f)
    small = b[fin & (np.abs(f) <= 448)]
    nz = b[fin & (f != 0)]
    H = 16
    rows = np.zeros((small.size + nz.size + 2, H), np.uint16)
    rows[:small.size, 0] = synth.to_bf16(np.float32([448.0]))[0]
    rows[:small.size, 1] = small
    rows[small.size:small.size + nz.size, 0] = nz
    rows[-1, 1::2] = 0x8000
    ref = oracle.quantize_fp8(rows)
    V = rows.shape[0]
    L = harness.to_dev_bf16(rows)
    q = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    s = torch.empty(V, dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    import mtp_draft_head_embed_amd as mtp
    mtp.mtp_quantize_head_fp8(L, V, H, q, s, ws)
    qg, sg = q.cpu().numpy(), s.cpu().numpy()
    badq = np.nonzero((qg != ref[0]).any(axis=1))[0]
    assert badq.size == 0, [(hex(rows[i, 0]), hex(rows[i, 1]), qg[i, :2], ref[0][i, :2]) for i in badq[:5]]
    bads = np.nonzero(sg.view(np.uint32) != ref[1].view(np.uint32))[0]
    assert bads.size == 0, [(hex(rows[i, 0]), sg[i], ref[1][i]) for i in bads[:5]]


def _midpoint_rows(amax_lo, amax_hi, width=2.0 ** -12):
    """Rows [a, w1..w15] (|w| <= a, so the scale is fl32(a / 448)) whose
    quotients w / s lie within `width` of an E4M3 rounding midpoint, measured
    in units of the code spacing: exact ties where s has few significant bits,
    near ties (a few float32 units off) elsewhere, and some just outside the
    window the kernel hands to the division."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    fin = np.isfinite(f) & (f != 0)
    avals = b[fin & (f >= amax_lo) & (f < amax_hi)]
    rows = []
    for a16 in avals:
        a = np.float64(np.float32((np.uint32(a16) << 16).view(np.float32)))
        s = np.float64(np.float32(a) / np.float32(448.0))
        ws = b[fin & (np.abs(f) <= a)]
        qv = np.abs(f[fin & (np.abs(f) <= a)].astype(np.float64) / s)
        nrm = qv >= 2.0 ** -6
        e = np.floor(np.log2(np.where(nrm, qv, 1.0)))
        k = np.where(nrm, (qv / 2.0 ** e - 1.0) * 16.0, qv * 1024.0)  # midpoints at odd k
        d = np.abs(k - (2.0 * np.floor(k / 2.0) + 1.0))
        pick = ws[(d < width) & (qv > 0)]
        for i in range(0, pick.size, 15):
            r = np.zeros(16, np.uint16)
            r[0] = a16
            r[1:1 + pick[i:i + 15].size] = pick[i:i + 15]
            rows.append(r)
    return np.array(rows, np.uint16)


def test_quantiser_midpoint_quotients():
    """Scales that are not powers of two (so 1/s is inexact) with quotients at
    or next to E4M3 rounding midpoints, including rows on both sides of the
    scale range where the kernel divides every element: codes and scales
    bit-exact against the oracle."""
    _say("\n[quantiser] near-midpoint quotients")
    rows = np.concatenate([_midpoint_rows(448.0, 896.0), _midpoint_rows(1.0, 2.0),
                           _midpoint_rows(2.0 ** -112, 2.0 ** -110)])
    assert rows.shape[0] > 500
    ref = oracle.quantize_fp8(rows)
    V, H = rows.shape
    import mtp_draft_head_embed_amd as mtp
    q = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    s = torch.empty(V, dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    mtp.mtp_quantize_head_fp8(harness.to_dev_bf16(rows), V, H, q, s, ws)
    qg, sg = q.cpu().numpy(), s.cpu().numpy()
    bad = np.argwhere(qg != ref[0])
    assert bad.size == 0, [(hex(rows[i, 0]), hex(rows[i, j]), hex(qg[i, j]), hex(ref[0][i, j]))
                           for i, j in bad[:5]]
    assert np.array_equal(sg.view(np.uint32), ref[1].view(np.uint32))


def test_stream_read_probe():
    """The streaming-read probe (a measurement aid) runs over a ragged-size
    buffer and leaves its output alone when the folded words do not match."""
    import mtp_draft_head_embed_amd as mtp
    buf = torch.zeros((1 << 20) + 48, dtype=torch.uint8, device="cuda")
    out = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    for per_cu in (1, 2, 16):
        mtp.mtp_probe_stream_read(buf, out, per_cu)
    torch.cuda.synchronize()
    assert int(out.item()) == 7


def test_fp8_convert_probe():
    """The hardware FP32 -> E4M3FN convert the quantiser encodes with rounds
    to nearest, ties to even, on every float of magnitude <= 448."""
    import mtp_draft_head_embed_amd as mtp
    res = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    mtp.mtp_probe_fp8_convert(res)
    torch.cuda.synchronize()
    bad, checked = (int(v) for v in res.cpu().numpy().view(np.uint32))
    assert checked == 2 * (0x43E00000 + 1)
    assert bad == 0, bad


def test_quantiser_nonfinite():
    import mtp_draft_head_embed_amd as mtp
    for bad in (0x7F80, 0xFF80, 0x7FC0):
        rows = np.zeros((5, 32), np.uint16)
        rows[3, 7] = bad
        L = harness.to_dev_bf16(rows)
        q = torch.empty((5, 32), dtype=torch.uint8, device="cuda")
        s = torch.empty(5, dtype=torch.float32, device="cuda")
        ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
        with pytest.raises(mtp.MtpError) as ei:
            mtp.mtp_quantize_head_fp8(L, 5, 32, q, s, ws)
        assert ei.value.status == mtp.MTP_ERR_NONFINITE
    # and a clean matrix afterwards reports success (the flag is cleared)
    rows = synth.normal_bf16(5, 32, 1, "lm_head", 0.0, 0.02)
    mtp.mtp_quantize_head_fp8(harness.to_dev_bf16(rows), 5, 32, q, s, ws)


@pytest.mark.parametrize("H", [512, 1024])
def test_invalid_tokens_and_no_logits(H):
    """tokens >= V give MTP_DRAFT_INVALID for that sequence only; skipping the
    logits output leaves the drafts unchanged (H = 512: the concat rows are
    written first; H = 1024: the fused front gathers in its prologue)."""
    _say(f"\n[invalid tokens] H={H}")
    cfg = synth.custom(H, 3000, 4, 40)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    tokens[1] = 3000
    tokens[3] = 0xFFFFFFFF
    dw = harness.upload(wts)
    d, lg = harness.run_draft(dw, tokens, hidden)
    assert d[1] == 0xFFFFFFFF and d[3] == 0xFFFFFFFF
    for b in (0, 2):
        r = oracle.draft(wts, int(tokens[b]), hidden[b])
        rep = harness.compare_sequence(b, r["o"], lg[b], int(d[b]), r["draft"], harness.TOL_BF16)
        assert rep.ok, rep
    d2, _ = harness.run_draft(dw, tokens, hidden, with_logits=False)
    assert np.array_equal(d, d2)


def test_determinism_repeat():
    cfg = synth.custom(1024, 20000, 2, 41)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    dw = harness.upload(wts)
    q, s = harness.quantize_dev(dw)
    for fp8 in (None, (q, s)):
        a = harness.run_draft(dw, tokens, hidden, fp8=fp8)
        for _ in range(3):
            b = harness.run_draft(dw, tokens, hidden, fp8=fp8)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_front_and_head_entry_points():
    """mtp_front's x against the oracle's FP64 x (final rounding plus the
    FP32 summation bound, almost all bit-equal), then mtp_head_* on the oracle's own
    x against the oracle head."""
    import mtp_draft_head_embed_amd as mtp
    cfg = synth.custom(1536, 9000, 3, 42)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    dw = harness.upload(wts)
    B, H, V = 3, 1536, 9000
    tk = torch.from_numpy(tokens.view(np.int32)).cuda()
    hd = harness.to_dev_bf16(hidden)
    x = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
    ws = mtp.new_workspace(H, V, B)
    mtp.mtp_front(dw.w, B, tk, hd, x, ws)
    torch.cuda.synchronize()
    xg = harness.bf16_bits(x)
    q, s = harness.quantize_dev(dw)
    qref = oracle.quantize_fp8(wts["lm_head"])
    xs = []
    for b in range(B):
        r = oracle.draft(wts, int(tokens[b]), hidden[b])
        xs.append(r["x"])
        harness.check_eh_proj_rows(xg[b:b + 1], r["x_unrounded"][None], r["concat"][None],
                                   r["concat_unrounded"][None], wts["eh_proj"])
    xo = harness.to_dev_bf16(np.stack(xs))
    for fp8 in (False, True):
        dr = torch.empty(B, dtype=torch.int32, device="cuda")
        lg = torch.empty((B, V), dtype=torch.bfloat16, device="cuda")
        if fp8:
            mtp.mtp_head_fp8w(dw.w, q, s, B, xo, dr, lg, ws)
        else:
            mtp.mtp_head_bf16(dw.w, B, xo, dr, lg, ws)
        torch.cuda.synchronize()
        lgb = harness.bf16_bits(lg)
        d = dr.cpu().numpy().view(np.uint32)
        for b in range(B):
            xn = oracle.rmsnorm(xs[b], wts["head_norm_w"], wts["rms_eps"])
            o = (oracle.gemv_fp8(qref[0], qref[1], xn) if fp8 else oracle.gemv_bf16(wts["lm_head"], xn))
            od = oracle.argmax_bf16(oracle.bf16_from_f64(o))
            rep = harness.compare_sequence(b, o, lgb[b], int(d[b]), od,
                                           harness.TOL_FP8 if fp8 else harness.TOL_BF16)
            assert rep.ok, rep


# ----------------------------------------------------------------------------
# full-size configurations
# ----------------------------------------------------------------------------

@pytest.fixture(scope="module")
def large():
    cfg = synth.CONFIGS["large"]
    _say("\n[large] generating weights")
    wts = synth.make_weights(cfg)
    return cfg, wts


@pytest.mark.slow
def test_mid_bf16():
    cfg = synth.CONFIGS["mid"]
    _say("\n[mid] generating weights")
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    dw = harness.upload(wts)
    _, _, reps = _check_all(cfg, wts, tokens, hidden, dw)
    _say(f"[mid] {reps}")


@pytest.mark.slow
def test_large_bf16_and_fp8(large):
    cfg, wts = large
    tokens, hidden = synth.make_inputs(cfg)
    dw = harness.upload(wts)
    _, _, reps = _check_all(cfg, wts, tokens, hidden, dw)
    _say(f"[large bf16] {reps}")
    q, s = harness.quantize_dev(dw)
    ref = oracle.quantize_fp8(wts["lm_head"])
    assert np.array_equal(q.cpu().numpy(), ref[0])
    assert np.array_equal(s.cpu().numpy(), ref[1])
    _, _, reps = _check_all(cfg, wts, tokens, hidden, dw, (q, s), ref)
    _say(f"[large fp8] {reps}")


@pytest.mark.slow
def test_batched_fp8():
    """B = 16 distinct tokens, FP8 head (the batched configuration)."""
    cfg = synth.CONFIGS["batched"]
    _say("\n[batched] generating weights")
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    assert len(set(tokens.tolist())) == 16
    dw = harness.upload(wts)
    q, s = harness.quantize_dev(dw)
    ref = oracle.quantize_fp8(wts["lm_head"])
    assert np.array_equal(q.cpu().numpy(), ref[0])
    _, _, reps = _check_all(cfg, wts, tokens, hidden, dw, (q, s), ref)
    _say(f"[batched fp8] max err {max(r.max_err for r in reps):.4g}")


@pytest.mark.slow
def test_neartie_bf16_and_fp8():
    """Near-tie stress (H = 6144, V = 154880, B = 8, Student-t(3) hidden, 64
    planted ids per sequence within 1e-3 of the max).  BF16 head: every planted
    logit rounds to the same value, so the draft must be the lowest planted id.
    FP8 head: the same where the quantised planted rows still round to one BF16
    value; otherwise the near-max and self-consistency rules."""
    from tests import neartie
    cfg = synth.CONFIGS["neartie"]
    _say("\n[neartie] generating weights and planting")
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    nt = neartie.build(cfg, wts, tokens, hidden)
    neartie.verify(nt, wts, tokens, hidden)
    w2 = dict(wts)
    w2["lm_head"] = nt.lm_head
    dw = harness.upload(w2)
    d, lg = harness.run_draft(dw, tokens, hidden)
    mins = [min(p) for p in nt.planted]
    assert [int(v) for v in d] == mins
    _, _, reps = _check_all(cfg, w2, tokens, hidden, dw)
    q, s = harness.quantize_dev(dw)
    ref = oracle.quantize_fp8(nt.lm_head)
    assert np.array_equal(q.cpu().numpy(), ref[0])
    assert np.array_equal(s.cpu().numpy(), ref[1])
    d8, lg8, reps8 = _check_all(cfg, w2, tokens, hidden, dw, (q, s), ref)
    exact_fp8 = 0
    for b in range(cfg.batch):
        r = oracle.draft(w2, int(tokens[b]), hidden[b], fp8=ref)
        P = np.array(nt.planted[b])
        if np.all(r["logits"][P] == r["logits"][P[0]]) and r["draft"] == P.min():
            assert int(d8[b]) == P.min(), b
            exact_fp8 += 1
    _say(f"[neartie] BF16 drafts == lowest planted ids for all {cfg.batch}; "
         f"FP8 exact-tie sequences: {exact_fp8}/{cfg.batch}")


def test_concurrent_streams():
    """Calls on two streams at once, each with its own workspace and buffers
    (a B = 1 BF16 sweep, whose head deals its last rows from counters in its
    workspace, beside a B = 3 FP8 sweep on the tile kernels), issued in turn
    without synchronising: each stream's outputs equal the same call made
    alone, bit for bit.  The library keeps no state between calls, so
    overlapping calls share nothing but the weights they read."""
    import mtp_draft_head_embed_amd as mtp
    H, V = 1024, 20000
    _say(f"\n[streams] H={H} V={V}")
    cfg = synth.custom(H, V, 4, 71)
    wts = synth.make_weights(cfg)
    dw = harness.upload(wts)
    q, s = harness.quantize_dev(dw)
    tokens, hidden = synth.make_inputs(cfg)
    runs = []
    for B, fp8, lo in ((1, False, 0), (3, True, 1)):
        tok, hid = tokens[lo:lo + B], hidden[lo:lo + B]
        tk = torch.from_numpy(tok.astype(np.uint32).view(np.int32)).cuda()
        hd = harness.to_dev_bf16(hid)
        dr = torch.empty(B, dtype=torch.int32, device="cuda")
        lg = torch.full((B, V), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = mtp.new_workspace(H, V, B)
        runs.append((B, fp8, tok, hid, tk, hd, dr, lg, ws, torch.cuda.Stream()))
    torch.cuda.synchronize()
    for _ in range(8):
        for B, fp8, _t, _h, tk, hd, dr, lg, ws, st in runs:
            if fp8:
                mtp.mtp_draft_fp8w(dw.w, q, s, B, tk, hd, dr, lg, ws, st)
            else:
                mtp.mtp_draft_bf16(dw.w, B, tk, hd, dr, lg, ws, st)
    torch.cuda.synchronize()
    for B, fp8, tok, hid, tk, hd, dr, lg, ws, st in runs:
        d_e, l_e = harness.run_draft(dw, tok, hid, fp8=(q, s) if fp8 else None)
        assert np.array_equal(dr.cpu().numpy().view(np.uint32), d_e), (B, fp8)
        assert np.array_equal(harness.bf16_bits(lg), l_e), (B, fp8)


@pytest.mark.parametrize("B,H", [(1, 1024), (3, 1024), (1, 6144)])
def test_graph_capture_replay(B, H):
    """A captured draft call replays correctly: new inputs copied into the
    captured buffers between replays (with eager work and synchronisation in
    between), every replay checked against an eager call on its own buffers
    and, for one replay, against the oracle.  At B = 1, H = 6144 the BF16 head
    deals its last passes of rows from counters the captured eh_proj clears;
    at B = 3 the tile head deals its last tiles from counters the captured
    sum-and-norm clears."""
    import mtp_draft_head_embed_amd as mtp
    _say(f"\n[graph] B={B} H={H}")
    V = 20000
    cfg = synth.custom(H, V, B, 60 + B)
    wts = synth.make_weights(cfg)
    dw = harness.upload(wts)
    q, s = harness.quantize_dev(dw)
    tk = torch.zeros(B, dtype=torch.int32, device="cuda")
    hd = torch.zeros((B, H), dtype=torch.bfloat16, device="cuda")
    ws = mtp.new_workspace(H, V, B)
    outs = {}
    graphs = {}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for path in ("bf16", "fp8"):
        dr = torch.empty(B, dtype=torch.int32, device="cuda")
        lg = torch.empty((B, V), dtype=torch.bfloat16, device="cuda")
        outs[path] = (dr, lg)
        with torch.cuda.stream(side):  # warm-up outside the capture
            if path == "fp8":
                mtp.mtp_draft_fp8w(dw.w, q, s, B, tk, hd, dr, lg, ws)
            else:
                mtp.mtp_draft_bf16(dw.w, B, tk, hd, dr, lg, ws)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            if path == "fp8":
                mtp.mtp_draft_fp8w(dw.w, q, s, B, tk, hd, dr, lg, ws)
            else:
                mtp.mtp_draft_bf16(dw.w, B, tk, hd, dr, lg, ws)
        graphs[path] = g
    torch.cuda.synchronize()
    for trial in range(3):
        tcfg = synth.custom(H, V, B, 600 + 10 * B + trial)
        tokens, hidden = synth.make_inputs(tcfg)
        tk.copy_(torch.from_numpy(tokens.view(np.int32)))
        hd.copy_(harness.to_dev_bf16(hidden))
        _ = (hd.float() * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        for path in ("bf16", "fp8"):
            graphs[path].replay()
            torch.cuda.synchronize()
            d_g = outs[path][0].cpu().numpy().view(np.uint32).copy()
            l_g = harness.bf16_bits(outs[path][1])
            d_e, l_e = harness.run_draft(dw, tokens, hidden, fp8=(q, s) if path == "fp8" else None)
            assert np.array_equal(d_g, d_e), (trial, path)
            assert np.array_equal(l_g, l_e), (trial, path)
            if trial == 1:
                ref = oracle.quantize_fp8(wts["lm_head"]) if path == "fp8" else None
                for b in range(B):
                    r = oracle.draft(wts, int(tokens[b]), hidden[b], fp8=ref)
                    rep = harness.compare_sequence(b, r["o"], l_g[b], int(d_g[b]), r["draft"],
                                                   harness.TOL_FP8 if ref else harness.TOL_BF16)
                    assert rep.ok, rep


@pytest.mark.slow
def test_head_logit_batches():
    """The single-sequence heads write their logits from LDS 128 rows per wave
    at a time: at H = 4608 (the same kernel instantiations as H = 6144, one
    row per pass BF16 and two FP8) and V = 300 000 every wave holds about 146
    rows, so each writes one batch inside its loop and the rest after it.
    Every logit of both heads, with and without the logits buffer, against the
    oracle."""
    H, V = 4608, 300000
    _say(f"\n[logit batches] H={H} V={V}")
    cfg = synth.custom(H, V, 1, 75)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    dw = harness.upload(wts)
    d, _, _ = _check_all(cfg, wts, tokens, hidden, dw)
    d0, _, _ = _check_all(cfg, wts, tokens, hidden, dw, with_logits=False)
    assert np.array_equal(d, d0)
    q, s = harness.quantize_dev(dw)
    ref = oracle.quantize_fp8(wts["lm_head"])
    d8, _, _ = _check_all(cfg, wts, tokens, hidden, dw, (q, s), ref)
    d80, _, _ = _check_all(cfg, wts, tokens, hidden, dw, (q, s), ref, with_logits=False)
    assert np.array_equal(d8, d80)


@pytest.mark.slow
@pytest.mark.parametrize("B", [1, 2])
def test_max_vocab(B):
    """The largest vocabulary the ABI accepts (2^24 rows) at the smallest
    hidden size: the longest per-wave row ranges on both kernel families."""
    import mtp_draft_head_embed_amd as mtp
    V, H = 1 << 24, 16
    assert mtp.mtp_workspace_bytes(H, V, B) > 0 and mtp.mtp_workspace_bytes(H, V + 1, B) == 0
    _say(f"\n[max vocab] V={V} H={H} B={B}")
    cfg = synth.custom(H, V, B, 70 + B)
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    tokens[-1] = V - 1  # the last embedding row
    dw = harness.upload(wts)
    _check_all(cfg, wts, tokens, hidden, dw)
    q, s = harness.quantize_dev(dw)
    ref = oracle.quantize_fp8(wts["lm_head"])
    assert np.array_equal(q.cpu().numpy(), ref[0])
    assert np.array_equal(s.cpu().numpy(), ref[1])
    _check_all(cfg, wts, tokens, hidden, dw, (q, s), ref)
