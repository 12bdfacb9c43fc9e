"""The eh_proj row checker (tests/harness.py, `check_eh_proj_rows`) on the
CPU.  It accepts an FP32 evaluation of the same rows done the way the library
does it: the norms in FP32 (so a few concat entries may round the other way)
and the products summed in FP32 in 32-column blocks, including a row that
nearly cancels.  It rejects the plausible mistakes: a dropped concat term, rows
swapped, a wrong token, and one wrong 16-column block at H = 6144."""
import numpy as np
import pytest

import oracle
import synth

harness = pytest.importorskip("tests.harness")


def _rows(H, V, T, seed):
    cfg = synth.custom(H, V, T + 1, seed)
    w = synth.make_weights(cfg)
    tokens, hid = synth.make_inputs(cfg)
    hiddens = np.ascontiguousarray(hid[:T])
    return w, tokens, hiddens, oracle.context_rows(w, tokens, hiddens)


def _fp32_norm(x_bits, w_bits, eps, recip=True):
    """BF16(x * w / sqrt(mean(x^2) + eps)) evaluated in float32 (numpy's
    pairwise sum of squares), the way a GPU norm is computed: x * w times the
    rounded reciprocal of the root (the library's form), or divided by it."""
    x = synth.from_bf16(x_bits)
    w = synth.from_bf16(w_bits)
    ss = np.sum(x * x, dtype=np.float32)
    r = np.sqrt(ss / np.float32(x.size) + np.float32(eps), dtype=np.float32)
    if recip:
        return synth.to_bf16((x * w) * (np.float32(1.0) / r))
    return synth.to_bf16((x * w) / r)


def _fp32_concat(w, tokens, hiddens, recip=True):
    """The concat rows of the context rows (row r: tokens[r + 1], hiddens[r])
    with FP32 norms."""
    rows = []
    for r in range(hiddens.shape[0]):
        e = w["embed"][int(tokens[r + 1])]
        rows.append(np.concatenate([_fp32_norm(e, w["enorm_w"], w["rms_eps"], recip),
                                    _fp32_norm(hiddens[r], w["hnorm_w"], w["rms_eps"], recip)]))
    return np.stack(rows)


def _fp32_eval(concat, eh_proj):
    """BF16 of an FP32 sum of the products: each 32-column block summed
    exactly and rounded once to FP32 (one matrix-core instruction), the blocks
    added in order in FP32."""
    c = harness.bits_to_f64(concat)
    W = harness.bits_to_f64(eh_proj)
    K = c.shape[1]
    acc = np.zeros((c.shape[0], W.shape[0]), dtype=np.float32)
    for k0 in range(0, K, 32):
        acc = (acc + (c[:, k0:k0 + 32] @ W[:, k0:k0 + 32].T).astype(np.float32)).astype(np.float32)
    return oracle.bf16_from_f64(acc.astype(np.float64))


def _check(xg, ref, w):
    return harness.check_eh_proj_rows(xg, ref["x_unrounded"], ref["concat"],
                                      ref["concat_unrounded"], w["eh_proj"])


def test_fp32_norm_flips_only_where_the_model_allows():
    """Every concat entry of an FP32 norm either equals the oracle's or is one
    the flip model marks (its unrounded value within the FP32 error of a BF16
    rounding boundary); and the model marks only a small share."""
    w, tokens, hiddens, ref = _rows(1024, 3000, 48, 85)
    delta = harness.concat_flip_delta(ref["concat"], ref["concat_unrounded"])
    flipped = 0
    for recip in (True, False):
        c32 = _fp32_concat(w, tokens, hiddens, recip)
        diff = c32 != ref["concat"]
        flipped += int(diff.sum())
        assert np.all(delta[diff] > 0), (recip, np.argwhere(diff & (delta == 0))[:5])
        # the flipped value is the neighbour the model names
        assert np.all(np.abs(harness.bits_to_f64(c32) - harness.bits_to_f64(ref["concat"]))[diff]
                      == delta[diff])
    assert flipped > 0  # the emulation does round some flagged entries the other way
    assert np.mean(delta > 0) < 0.01


def test_accepts_fp32_sums_with_cancellation():
    # H=256, 64 rows, seed 83: row 56 column 3 sums to about 1e-6 of sum |terms|
    w, tokens, hiddens, ref = _rows(256, 3000, 64, 83)
    m = np.abs(harness.bits_to_f64(ref["concat"])) @ np.abs(harness.bits_to_f64(w["eh_proj"])).T
    assert np.min(np.abs(ref["x_unrounded"]) / m) < 1e-5
    _check(_fp32_eval(ref["concat"], w["eh_proj"]), ref, w)
    _check(_fp32_eval(_fp32_concat(w, tokens, hiddens), w["eh_proj"]), ref, w)
    _check(ref["x"], ref, w)


def test_rejects_mistakes():
    w, tokens, hiddens, ref = _rows(256, 3000, 40, 84)
    dropped = ref["concat"].copy()
    dropped[:, 17] = 0  # one concat entry lost in every row
    with pytest.raises(AssertionError):
        _check(_fp32_eval(dropped, w["eh_proj"]), ref, w)
    swapped = ref["x"].copy()
    swapped[[3, 4]] = swapped[[4, 3]]
    with pytest.raises(AssertionError):
        _check(swapped, ref, w)
    # a row built from the neighbouring token (tokens[r] instead of tokens[r + 1])
    c = oracle.front(w["embed"], int(tokens[5]), hiddens[5], w["enorm_w"], w["hnorm_w"],
                     float(w["rms_eps"]))
    off_by_one = ref["x"].copy()
    off_by_one[5] = oracle.bf16_from_f64(oracle.gemv_bf16(w["eh_proj"], c))
    with pytest.raises(AssertionError):
        _check(off_by_one, ref, w)


def test_large_hidden_tight_bound_and_wrong_block():
    """H = 6144 (K = 12288): the FP32 evaluation passes with a median bound of
    a few ulps of x, and one wrong 16-column block of the concat (zeroed, or a
    copy of its neighbour) in every row fails."""
    w, tokens, hiddens, ref = _rows(6144, 2000, 3, 86)
    c32 = _fp32_concat(w, tokens, hiddens)
    st = _check(_fp32_eval(c32, w["eh_proj"]), ref, w)
    assert st["median_bound_ulps"] < 4, st
    for k0 in (0, 4096, 12288 - 16):
        bad = c32.copy()
        bad[:, k0:k0 + 16] = 0
        with pytest.raises(AssertionError):
            _check(_fp32_eval(bad, w["eh_proj"]), ref, w)
    bad = c32.copy()
    bad[:, 6144:6160] = c32[:, 6160:6176]
    with pytest.raises(AssertionError):
        _check(_fp32_eval(bad, w["eh_proj"]), ref, w)


def test_accepts_a_flipped_concat_entry_only_where_it_can_flip():
    """A flagged entry moved to its neighbour keeps its row inside the bound;
    flipping entries the model does not flag, in every row, is rejected."""
    w, tokens, hiddens, ref = _rows(256, 3000, 64, 83)
    delta = harness.concat_flip_delta(ref["concat"], ref["concat_unrounded"])
    flagged = np.argwhere(delta > 0)
    assert flagged.shape[0] > 0
    c = ref["concat"].copy()
    for r, k in flagged[:10]:
        u = ref["concat_unrounded"][r, k]
        key = harness.bf16_order_key(c[r:r + 1, k:k + 1])[0, 0]
        cv = harness.bits_to_f64(c[r:r + 1, k:k + 1])[0, 0]
        c[r, k] = harness._bf16_from_key(np.array([key + (1 if u >= cv else -1)]))[0]
    _check(_fp32_eval(c, w["eh_proj"]), ref, w)
    bad = ref["concat"].copy()
    for r in range(bad.shape[0]):
        ks = [k for k in range(bad.shape[1]) if delta[r, k] == 0 and bad[r, k] & 0x7FFF][:8]
        key = harness.bf16_order_key(bad[r, ks])
        bad[r, ks] = harness._bf16_from_key(key + np.where(key >= 0, 1, -1))
    with pytest.raises(AssertionError):
        _check(_fp32_eval(bad, w["eh_proj"]), ref, w)
