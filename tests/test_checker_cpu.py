"""The eh_proj row checker (tests/harness.py, `check_eh_proj_rows`) on the
CPU: it accepts an FP32 evaluation of the same rows (any summation order, the
way the GPU sums), including a row that nearly cancels, and rejects the
plausible mistakes (a dropped concat term, rows swapped, a wrong token)."""
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


def _fp32_eval(concat, eh_proj):
    """BF16(FP32 sum) of the same products, summed in FP32 by numpy."""
    c = harness.bits_to_f64(concat).astype(np.float32)
    W = harness.bits_to_f64(eh_proj).astype(np.float32)
    return oracle.bf16_from_f64((c @ W.T).astype(np.float64))


def test_accepts_fp32_sums_with_cancellation():
    # H=256, 64 rows, seed 83: row 56 column 3 sums to about 1e-6 of sum |terms|
    w, tokens, hiddens, ref = _rows(256, 3000, 64, 83)
    m = np.abs(harness.bits_to_f64(ref["concat"])) @ np.abs(harness.bits_to_f64(w["eh_proj"])).T
    assert np.min(np.abs(ref["x_unrounded"]) / m) < 1e-5
    xg = _fp32_eval(ref["concat"], w["eh_proj"])
    harness.check_eh_proj_rows(xg, ref["x_unrounded"], ref["concat"], w["eh_proj"])
    harness.check_eh_proj_rows(ref["x"], ref["x_unrounded"], ref["concat"], w["eh_proj"])


def test_rejects_mistakes():
    w, tokens, hiddens, ref = _rows(256, 3000, 40, 84)
    args = (ref["x_unrounded"], ref["concat"], w["eh_proj"])
    dropped = ref["concat"].copy()
    dropped[:, 17] = 0  # one concat entry lost in every row
    with pytest.raises(AssertionError):
        harness.check_eh_proj_rows(_fp32_eval(dropped, w["eh_proj"]), *args)
    swapped = ref["x"].copy()
    swapped[[3, 4]] = swapped[[4, 3]]
    with pytest.raises(AssertionError):
        harness.check_eh_proj_rows(swapped, *args)
    # a row built from the neighbouring token (tokens[r] instead of tokens[r + 1])
    c = oracle.front(w["embed"], int(tokens[5]), hiddens[5], w["enorm_w"], w["hnorm_w"],
                     float(w["rms_eps"]))
    off_by_one = ref["x"].copy()
    off_by_one[5] = oracle.bf16_from_f64(oracle.gemv_bf16(w["eh_proj"], c))
    with pytest.raises(AssertionError):
        harness.check_eh_proj_rows(off_by_one, *args)


def test_accepts_a_flipped_concat_entry():
    """A concat entry one ulp away (the FP32 norm rounding the other way) keeps
    its row inside the bound."""
    w, tokens, hiddens, ref = _rows(256, 3000, 64, 83)
    c = ref["concat"].copy()
    for r, k in [(16, 100), (27, 300), (40, 5)]:
        c[r, k] += 1  # next BF16 magnitude
    harness.check_eh_proj_rows(_fp32_eval(c, w["eh_proj"]), ref["x_unrounded"], ref["concat"],
                               w["eh_proj"])
