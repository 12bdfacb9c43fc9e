"""Pins for the oracle's number formats: BF16 rounding and OCP E4M3FN.

The E4M3 drafting copy of lm_head is described in the `head_fp8` field doc of
metrale_model_arch/glm5next_mtp_head.rs; BF16 storage of every intermediate
(concat, x, logits) in the per-sequence scratch of the same page
(`Glm5NextMtpProposerState`).  The oracle's encoders are checked against hand
values, library routines and brute-force nearest-value searches.
"""
import math
import os

import numpy as np
import pytest
import torch

from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_table.txt")


def _golden():
    enc, dec = [], []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        kind, a, b = line.split()
        if kind == "encode":
            enc.append((float(eval(a)), int(b, 16)))
        else:
            dec.append((int(a, 16), float("nan") if b == "nan" else float(eval(b))))
    return enc, dec


def test_e4m3_hand_table(orc):
    enc, dec = _golden()
    assert len(enc) >= 20 and len(dec) >= 10
    for y, code in enc:
        assert orc.e4m3_encode(y) == code, (y, hex(code))
    for code, v in dec:
        got = orc.e4m3_decode(code)
        if math.isnan(v):
            assert math.isnan(got)
        else:
            assert got == v and math.copysign(1, got) == math.copysign(1, v), hex(code)


def test_e4m3_decode_all_codes(orc):
    """All 256 codes against a bit-construction decoder; 254 finite codes,
    strictly increasing magnitudes over 0x00..0x7E, sign symmetry."""
    vals = [orc.e4m3_decode(c) for c in range(256)]
    ref = [exact.e4m3_bits_value(c) for c in range(256)]
    finite = [v for v in vals if not math.isnan(v)]
    assert len(finite) == 254
    for c in range(256):
        if math.isnan(ref[c]):
            assert math.isnan(vals[c])
        else:
            assert vals[c] == ref[c]
    mags = vals[:0x7F]
    assert all(mags[i] < mags[i + 1] for i in range(0x7E))
    for c in range(0x7F):
        assert vals[c | 0x80] == -vals[c]


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    return b[np.isfinite(f)], f[np.isfinite(f)]


def test_e4m3_encode_exhaustive_bf16(orc):
    """Every finite BF16 value with |w| <= 448 (and the saturating rest)
    against a brute-force nearest-code search with ties to the even code."""
    _, f = _all_finite_bf16()
    got = np.array([orc.e4m3_encode(float(v)) for v in f], dtype=np.uint8)
    want = np.concatenate([exact.e4m3_brute_vec(f[i:i + 4096])
                           for i in range(0, f.size, 4096)])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(f[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_e4m3_encode_random_f32(orc):
    """fl32(w / s) is a general binary32, not only a BF16 value: random float32
    magnitudes spread over the whole E4M3 range, plus exact midpoints."""
    g = np.random.default_rng(7)
    e = g.uniform(-12, 9.2, size=20000)
    y = (np.sign(g.standard_normal(20000)) * 2.0 ** e).astype(np.float32)
    mags = np.array([exact.e4m3_bits_value(m) for m in range(0x7F)])
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    y = np.concatenate([y, mids, -mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1000))])
    got = np.array([orc.e4m3_encode(float(v)) for v in y], dtype=np.uint8)
    want = np.concatenate([exact.e4m3_brute_vec(y[i:i + 4096]) for i in range(0, y.size, 4096)])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(y[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_bf16_from_double_matches_torch_on_float32(orc):
    """For binary32 inputs a one-step double -> BF16 rounding must equal the
    library float32 -> bfloat16 conversion (round to nearest even)."""
    g = np.random.default_rng(3)
    bits = g.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    # plus exact midpoints between neighbouring BF16 values
    b = g.integers(0, 0x7F00, size=5000).astype(np.uint32)
    mid = ((b << 16) | 0x8000).view(np.float32)
    f = np.concatenate([f, mid, -mid])
    got = orc.bf16_from_f64(f.astype(np.float64))
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(f[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_bf16_from_double_single_rounding(orc):
    """Doubles that are not binary32 values: the result is the nearest BF16 by
    exact search; a float32 detour (double rounding) would fail some of these."""
    g = np.random.default_rng(11)
    xs = list(g.standard_normal(3000) * 10.0 ** g.uniform(-30, 30, 3000))
    # just above a BF16 midpoint by less than a float32 ulp: double -> float ->
    # bf16 lands on the midpoint and rounds to even, the one-step rounding up.
    for base in [1.0, 1.5, 3.25, 100.0, 7.0e-3]:
        b = int(np.float32(base).view(np.uint32)) >> 16
        mid = float(exact.bf16_exact(b)) + float(exact.bf16_exact(b + 1) - exact.bf16_exact(b)) / 2
        xs += [mid + mid * 2.0 ** -40, mid - mid * 2.0 ** -40, mid]
    got = orc.bf16_from_f64(np.array(xs))
    from fractions import Fraction
    for x, gbits in zip(xs, got):
        assert int(gbits) == exact.bf16_nearest(Fraction(x)), x


def test_bf16_signed_zero_and_subnormal(orc):
    got = orc.bf16_from_f64(np.array([0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134,
                                      -(2.0 ** -140)]))
    assert [int(v) for v in got] == [0x0000, 0x8000, 0x0001, 0x0000, 0x0002, 0x8000]
