"""Pins for the oracle's draft-sweep steps, each against something other than
itself: closed forms, exact rationals (BF16 values are dyadic, so products and
sums are exact in ``Fraction``; square roots are taken to 80 digits), library
routines and invariants.

Steps follow metrale_model_arch/glm5next_mtp_head.rs (module doc: the draft
formula; ``forward_one``: embed row by pointer, enorm, hnorm, concat, eh_proj,
``shared_head.norm``, lm_head, argmax; ``head_fp8``: the FP8 E4M3 copy) and
metrale_model_arch/glm5next_layer/mod.rs (invariants: ``rms_norm_vanilla`` is
``x * w / rms``, never ``1 + w``).
"""
from decimal import Decimal
from fractions import Fraction

import numpy as np
import pytest

from synth import to_bf16
from tests import exact

ONE = 0x3F80  # BF16 1.0
EPS = 1e-6
EPS_EXACT = Fraction(float(np.float32(EPS)))


def bf(vals):
    return to_bf16(np.asarray(vals, dtype=np.float32))


def rand_bf16(g, shape, std=1.0, mean=0.0):
    return to_bf16((g.standard_normal(shape) * std + mean).astype(np.float32))


def exact_norm(x, w, eps_exact=EPS_EXACT):
    """Vanilla RMSNorm of BF16 vectors, exact up to the 80-digit square root,
    rounded by nearest-value search."""
    xs = [exact.bf16_exact(v) for v in x]
    ws = [exact.bf16_exact(v) for v in w]
    S = sum(v * v for v in xs) / len(xs) + eps_exact
    r = exact.dec_sqrt(S)
    out = []
    for a, b in zip(xs, ws):
        p = a * b
        out.append(exact.bf16_nearest(Decimal(p.numerator) / Decimal(p.denominator) / r))
    return np.array(out, dtype=np.uint16)


# ----------------------------------------------------------------------------
# rms_norm_vanilla
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("c", [1.0, 0.5, 3.0, 0.001, 250.0])
def test_norm_constant_vector(orc, c):
    """w = 1, x = c * ones: every output is BF16(c / sqrt(c^2 + eps))."""
    H = 64
    x = bf([c] * H)
    cc = exact.bf16_exact(int(x[0]))
    want = exact.bf16_nearest(Decimal(cc.numerator) / Decimal(cc.denominator)
                              / exact.dec_sqrt(cc * cc + EPS_EXACT))
    out = orc.rmsnorm(x, np.full(H, ONE, np.uint16), EPS)
    assert np.all(out == want)
    if c == 1.0:
        assert int(out[0]) == ONE


def test_norm_one_hot(orc):
    """w = 1, x = a e_k: out_k = a / sqrt(a^2/H + eps) (a = 1, H = 256 -> 16.0),
    every other output exactly +0 -- this also fixes mean (not sum) of squares."""
    H, k = 256, 37
    x = np.zeros(H, np.uint16)
    x[k] = ONE
    out = orc.rmsnorm(x, np.full(H, ONE, np.uint16), EPS)
    assert int(out[k]) == int(bf([16.0])[0])
    assert np.all(np.delete(out, k) == 0)


def test_norm_zero_weight_lane(orc):
    """A w = 0 lane gives exactly 0; a (1 + w) norm would give x / rms there."""
    g = np.random.default_rng(1)
    H = 128
    x = rand_bf16(g, H)
    w = rand_bf16(g, H, 0.1, 1.0)
    w[5] = 0
    w[77] = 0x8000  # -0.0
    out = orc.rmsnorm(x, w, EPS)
    assert exact.bf16_exact(int(out[5])) == 0 and exact.bf16_exact(int(out[77])) == 0
    assert np.count_nonzero(exact_norm(x, w) != out) == 0


@pytest.mark.parametrize("H", [1, 2, 5, 16])
def test_norm_exact_rationals(orc, H):
    g = np.random.default_rng(100 + H)
    for trial in range(20):
        x = rand_bf16(g, H, 10.0 ** g.uniform(-3, 2))
        w = rand_bf16(g, H, 0.3, 1.0)
        assert np.array_equal(orc.rmsnorm(x, w, EPS), exact_norm(x, w)), trial


@pytest.mark.parametrize("H", [1, 2, 5, 16])
def test_norm_unrounded_exact_rationals(orc, H):
    """The norm's FP64 values before rounding: within 1e-14 (relative) of the
    exact x_j w_j / sqrt(mean(x^2) + eps), and rounding them gives the
    rounded norm's outputs bit for bit."""
    g = np.random.default_rng(300 + H)
    for trial in range(20):
        x = rand_bf16(g, H, 10.0 ** g.uniform(-3, 2))
        w = rand_bf16(g, H, 0.3, 1.0)
        u = orc.rmsnorm_unrounded(x, w, EPS)
        xs = [exact.bf16_exact(v) for v in x]
        ws = [exact.bf16_exact(v) for v in w]
        r = exact.dec_sqrt(sum(v * v for v in xs) / len(xs) + EPS_EXACT)
        for j in range(H):
            p = xs[j] * ws[j]
            want = Decimal(p.numerator) / Decimal(p.denominator) / r
            assert abs(Decimal(float(u[j])) - want) <= abs(want) * Decimal("1e-14"), (trial, j)
        assert np.array_equal(orc.bf16_from_f64(u), orc.rmsnorm(x, w, EPS)), trial


def test_norm_unrounded_closed_forms(orc):
    """w = 1, x = e_k at H = 256: 16 exactly at k, zeros elsewhere; w = 1,
    x = c * ones: c / sqrt(c^2 + eps) in every lane."""
    H, k = 256, 37
    x = np.zeros(H, np.uint16)
    x[k] = ONE
    u = orc.rmsnorm_unrounded(x, np.full(H, ONE, np.uint16), EPS)
    assert abs(u[k] - 16.0 / np.sqrt(1.0 + 256.0 * float(np.float32(EPS)))) < 1e-13
    assert np.all(np.delete(u, k) == 0.0)
    c = float(exact.bf16_exact(int(bf([3.0])[0])))
    u = orc.rmsnorm_unrounded(bf([3.0] * 64), np.full(64, ONE, np.uint16), EPS)
    assert np.allclose(u, c / np.sqrt(c * c + float(np.float32(EPS))), rtol=1e-15, atol=0)


def test_norm_eps_matters(orc):
    """A tiny row, where eps dominates: sqrt(mean(x^2) + eps), eps as f32."""
    H = 8
    x = bf([1e-4] * H)
    out = orc.rmsnorm(x, np.full(H, ONE, np.uint16), EPS)
    assert np.array_equal(out, exact_norm(x, np.full(H, ONE, np.uint16)))
    xv = float(exact.bf16_exact(int(x[0])))
    assert abs(float(exact.bf16_exact(int(out[0]))) - xv / np.sqrt(xv * xv + 1e-6)) < 0.01


# ----------------------------------------------------------------------------
# gather + concat + eh_proj
# ----------------------------------------------------------------------------

def _weights(g, H, V, unit_norms=False):
    w = {
        "embed": rand_bf16(g, (V, H), 0.5),
        "enorm_w": rand_bf16(g, H, 0.1, 1.0),
        "hnorm_w": rand_bf16(g, H, 0.1, 1.0),
        "eh_proj": rand_bf16(g, (H, 2 * H), 0.2),
        "head_norm_w": rand_bf16(g, H, 0.1, 1.0),
        "lm_head": rand_bf16(g, (V, H), 0.2),
        "rms_eps": EPS,
    }
    if unit_norms:
        for k in ("enorm_w", "hnorm_w", "head_norm_w"):
            w[k] = np.full(H, ONE, np.uint16)
    return w


def test_front_gather_and_bounds(orc):
    g = np.random.default_rng(2)
    H, V = 32, 50
    w = _weights(g, H, V)
    hid = rand_bf16(g, H)
    for tok in (0, V - 1, 17):
        c = orc.front(w["embed"], tok, hid, w["enorm_w"], w["hnorm_w"], EPS)
        assert np.array_equal(c[:H], exact_norm(w["embed"][tok], w["enorm_w"]))
        assert np.array_equal(c[H:], exact_norm(hid, w["hnorm_w"]))
        # the unrounded concat: same order, and it rounds to the concat
        u = orc.front_unrounded(w["embed"], tok, hid, w["enorm_w"], w["hnorm_w"], EPS)
        assert np.array_equal(orc.bf16_from_f64(u), c)
    assert orc.front(w["embed"], V, hid, w["enorm_w"], w["hnorm_w"], EPS) is None
    assert orc.front_unrounded(w["embed"], V, hid, w["enorm_w"], w["hnorm_w"], EPS) is None
    assert orc.front(w["embed"], 2 ** 32 - 1, hid, w["enorm_w"], w["hnorm_w"], EPS) is None


def test_concat_order_closed_form(orc):
    """eh_proj = [I | 0] gives x = enorm(embed[token]); [0 | I] gives hnorm(hidden)."""
    g = np.random.default_rng(3)
    H, V = 24, 40
    w = _weights(g, H, V)
    hid = rand_bf16(g, H)
    eye = np.zeros((H, 2 * H), np.uint16)
    eye[np.arange(H), np.arange(H)] = ONE
    w["eh_proj"] = eye
    r = orc.draft(w, 9, hid)
    assert np.array_equal(r["x"], exact_norm(w["embed"][9], w["enorm_w"]))
    eye2 = np.zeros((H, 2 * H), np.uint16)
    eye2[np.arange(H), H + np.arange(H)] = ONE
    w["eh_proj"] = eye2
    r = orc.draft(w, 9, hid)
    assert np.array_equal(r["x"], exact_norm(hid, w["hnorm_w"]))


def _exact_gemv(W, x):
    out = []
    for row in W:
        out.append(sum(exact.bf16_exact(a) * exact.bf16_exact(b) for a, b in zip(row, x)))
    return out


@pytest.mark.parametrize("n,k", [(1, 1), (3, 7), (8, 16), (13, 33)])
def test_gemv_exact_rationals(orc, n, k):
    """Unrounded oracle GEMV within the sequential-summation error bound of the
    exact rational result; BF16 rounding agrees with nearest-value search."""
    g = np.random.default_rng(n * 100 + k)
    W = rand_bf16(g, (n, k))
    x = rand_bf16(g, k)
    got = orc.gemv_bf16(W, x, nthreads=1)
    ex = _exact_gemv(W, x)
    for i in range(n):
        absum = sum(abs(exact.bf16_exact(a) * exact.bf16_exact(b)) for a, b in zip(W[i], x))
        bound = Fraction(max(k - 1, 0)) * Fraction(1, 2 ** 53) * absum * Fraction(11, 10)
        assert abs(Fraction(float(got[i])) - ex[i]) <= bound
    rounded = orc.bf16_from_f64(got)
    want = np.array([exact.bf16_nearest(v) for v in ex], dtype=np.uint16)
    assert np.array_equal(rounded, want)


def test_gemv_row_major_layout(orc):
    """W[i][j] multiplies x[j]: a non-square W with one-hot rows picks x at the
    given columns (a transposed read would pick other elements)."""
    g = np.random.default_rng(5)
    n, k = 5, 11
    x = rand_bf16(g, k)
    W = np.zeros((n, k), np.uint16)
    cols = [3, 0, 10, 7, 7]
    for i, j in enumerate(cols):
        W[i, j] = ONE
    got = orc.gemv_bf16(W, x)
    assert [float(v) for v in got] == [float(exact.bf16_exact(x[j])) for j in cols]


def test_gemv_thread_invariance(orc):
    g = np.random.default_rng(6)
    W = rand_bf16(g, (1001, 96))
    x = rand_bf16(g, 96)
    a = orc.gemv_bf16(W, x, nthreads=1)
    b = orc.gemv_bf16(W, x, nthreads=7)
    assert a.tobytes() == b.tobytes()


# ----------------------------------------------------------------------------
# head: BF16, FP8, argmax
# ----------------------------------------------------------------------------

def test_head_permutation(orc):
    """A permutation lm_head returns the permuted activation exactly."""
    g = np.random.default_rng(7)
    H = 40
    xn = rand_bf16(g, H)
    perm = g.permutation(H)
    L = np.zeros((H, H), np.uint16)
    L[np.arange(H), perm] = ONE
    o = orc.gemv_bf16(L, xn)
    assert np.array_equal(orc.bf16_from_f64(o), xn[perm])


def test_fp8_head_one_hot(orc):
    """One code per row: o_v = s_v * dec(c) * x_j, a single exact product."""
    g = np.random.default_rng(8)
    H, V = 32, 60
    x = rand_bf16(g, H)
    q = np.zeros((V, H), np.uint8)
    s = g.uniform(1e-4, 1e-1, V).astype(np.float32)
    cols = g.integers(0, H, V)
    codes = g.integers(0, 0x7F, V)
    codes[codes == 0x7F] = 0x7E
    sign = g.integers(0, 2, V) * 0x80
    q[np.arange(V), cols] = codes | sign
    o = orc.gemv_fp8(q, s, x)
    for v in range(V):
        want = (Fraction(float(s[v])) * Fraction(exact.e4m3_bits_value(int(q[v, cols[v]])))
                * exact.bf16_exact(x[cols[v]]))
        assert Fraction(float(o[v])) == want


def test_fp8_head_lossless_equals_bf16(orc):
    """Rows whose amax is 448 * 2^k and whose entries lie on the 2^k E4M3 grid
    quantise losslessly (s = 2^k), so the FP8 head's logits equal the BF16
    head's bit for bit."""
    g = np.random.default_rng(9)
    H, V = 64, 100
    k = -12
    mags = np.array([exact.e4m3_bits_value(m) for m in range(0x7F)])
    codes = g.integers(0, 0x7F, (V, H))
    vals = mags[codes] * np.where(g.integers(0, 2, (V, H)) == 1, -1.0, 1.0)
    vals[np.arange(V), g.integers(0, H, V)] = 448.0 * np.where(g.integers(0, 2, V) == 1, -1, 1)
    L = to_bf16((vals * 2.0 ** k).astype(np.float32))
    assert np.array_equal(exact_f32 := (L.astype(np.uint32) << 16).view(np.float32),
                          (vals * 2.0 ** k).astype(np.float32))
    qs = orc.quantize_fp8(L)
    assert qs is not None
    q, s = qs
    assert np.all(s == np.float32(2.0 ** k))
    x = rand_bf16(g, H)
    o8 = orc.gemv_fp8(q, s, x)
    o16 = orc.gemv_bf16(L, x)
    assert o8.tobytes() == o16.tobytes()


def test_argmax_lowest_index_and_signed_zero(orc):
    g = np.random.default_rng(10)
    for trial in range(50):
        n = int(g.integers(1, 3000))
        lg = rand_bf16(g, n, 2.0)
        m = lg.copy()
        # plant duplicate maxima at several places
        top = bf([50.0])[0]
        for p in g.choice(n, size=min(n, 4), replace=False):
            m[p] = top
        for arr in (lg, m):
            assert orc.argmax_bf16(arr) == int(np.argmax(exact_f := (arr.astype(np.uint32) << 16).view(np.float32)))
    for n in (1, 2, 1000):
        arr = np.full(n, bf([-1.0])[0], np.uint16)
        arr[0] = arr[-1] = bf([3.0])[0]
        assert orc.argmax_bf16(arr) == 0
    # -0 and +0 compare equal: the lower index wins
    arr = bf([-1.0, -0.0, 0.0, -2.0])
    assert orc.argmax_bf16(arr) == 1
    arr = bf([-1.0, 0.0, -0.0, -2.0])
    assert orc.argmax_bf16(arr) == 1


# ----------------------------------------------------------------------------
# FP8 quantiser
# ----------------------------------------------------------------------------

def _finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    ok = np.isfinite(f)
    return b[ok], f[ok]


def test_quant_rows_with_unit_scale_exhaustive(orc):
    """Rows [448, w] for every finite BF16 |w| <= 448 have s = 1 exactly, so
    q(w) is the brute-force nearest code (ties to even)."""
    b, f = _finite_bf16()
    sel = np.abs(f) <= 448
    b, f = b[sel], f[sel]
    L = np.stack([np.full(b.size, bf([448.0])[0], np.uint16), b], axis=1)
    q, s = orc.quantize_fp8(L)
    assert np.all(s == 1.0)
    assert np.all(q[:, 0] == 0x7E)
    want = np.concatenate([exact.e4m3_brute_vec(f[i:i + 4096]) for i in range(0, f.size, 4096)])
    assert np.array_equal(q[:, 1], want)


def test_quant_rows_scale_path_exhaustive(orc):
    """Rows [w, 0] for every finite nonzero BF16 w: the row max maps to the
    largest code of its sign, zero to 0x00, and s is the correctly rounded
    binary32 quotient |w| / 448 (within half an ulp of s)."""
    b, f = _finite_bf16()
    sel = f != 0
    b, f = b[sel], f[sel]
    L = np.stack([b, np.zeros(b.size, np.uint16)], axis=1)
    q, s = orc.quantize_fp8(L)
    assert np.all(q[:, 0] == np.where(f < 0, 0xFE, 0x7E))
    assert np.all(q[:, 1] == 0)
    a = np.abs(f).astype(np.float64)
    sd = s.astype(np.float64)
    # |s * 448 - a| <= 448 * half-ulp(s), ulp from the binary32 spacing at s
    ulp = np.spacing(s).astype(np.float64)
    assert np.all(np.abs(sd * 448.0 - a) <= 448.0 * ulp / 2)
    assert np.all(s > 0)


def test_quant_zero_and_nonfinite_rows(orc):
    L = bf([[0.0, -0.0, 0.0, -0.0], [1.0, 2.0, 3.0, 4.0]])
    q, s = orc.quantize_fp8(L)
    assert s[0] == 1.0 and list(q[0]) == [0x00, 0x80, 0x00, 0x80]
    for bad in (np.inf, -np.inf, np.nan):
        L2 = bf([[1.0, 2.0], [bad, 0.5]])
        if np.isnan(bad):
            L2[1, 0] = 0x7FC0
        assert orc.quantize_fp8(L2) is None


def test_quant_reconstruction_bound(orc):
    """dec(q) * s reproduces each weight within the E4M3 rounding bound:
    relative 2^-4 for normals, absolute 2^-10 * s for subnormals."""
    g = np.random.default_rng(12)
    V, H = 200, 96
    f = (g.standard_normal((V, H)) * 0.02).astype(np.float32)
    f[::7, 3] *= 300.0  # outliers set some rows' scale
    L = to_bf16(f)
    q, s = orc.quantize_fp8(L, nthreads=3)
    q1, s1 = orc.quantize_fp8(L, nthreads=1)
    assert np.array_equal(q, q1) and np.array_equal(s, s1)
    w = (L.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mags = np.array([exact.e4m3_bits_value(m) for m in range(0x7F)])
    dec = np.where(q >= 0x80, -mags[q & 0x7F], mags[q & 0x7F])
    rec = dec * s[:, None].astype(np.float64)
    err = np.abs(rec - w)
    bound = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)
    assert np.all((q & 0x7F).max(axis=1) == 0x7E)


# ----------------------------------------------------------------------------
# End to end
# ----------------------------------------------------------------------------

def test_end_to_end_closed_form(orc):
    """Unit norm weights, eh_proj = [I | 0], lm_head = [I_H ; 0]: logits are the
    twice-normed embedding row followed by zeros, and the draft is the position
    of that row's (clearly largest, positive) element."""
    g = np.random.default_rng(13)
    H, V = 48, 100
    w = _weights(g, H, V, unit_norms=True)
    eye = np.zeros((H, 2 * H), np.uint16)
    eye[np.arange(H), np.arange(H)] = ONE
    w["eh_proj"] = eye
    L = np.zeros((V, H), np.uint16)
    L[np.arange(H), np.arange(H)] = ONE
    w["lm_head"] = L
    for tok, k in ((5, 0), (60, 47), (99, 21)):
        row = (g.standard_normal(H) * 0.3).astype(np.float32)
        row[k] = 4.0
        w["embed"][tok] = to_bf16(row)
        r = orc.draft(w, tok, rand_bf16(g, H))
        assert r["draft"] == k
        x = exact_norm(w["embed"][tok], w["enorm_w"])
        assert np.array_equal(r["x"], x)
        assert np.array_equal(r["logits"][:H], exact_norm(x, w["head_norm_w"]))
        assert np.all(r["logits"][H:] == 0)


@pytest.mark.parametrize("seed", [21, 22])
def test_end_to_end_exact_tiny(orc, seed):
    """Tiny random sweep recomputed in exact arithmetic with nearest-value
    rounding at every BF16 storage point."""
    g = np.random.default_rng(seed)
    H, V = 8, 24
    w = _weights(g, H, V)
    hid = rand_bf16(g, H, 2.0)
    tok = int(g.integers(0, V))
    r = orc.draft(w, tok, hid)
    c = np.concatenate([exact_norm(w["embed"][tok], w["enorm_w"]), exact_norm(hid, w["hnorm_w"])])
    assert np.array_equal(r["concat"], c)
    x = np.array([exact.bf16_nearest(v) for v in _exact_gemv(w["eh_proj"], c)], np.uint16)
    assert np.array_equal(r["x"], x)
    xn = exact_norm(x, w["head_norm_w"])
    assert np.array_equal(r["xn"], xn)
    o = _exact_gemv(w["lm_head"], xn)
    lg = np.array([exact.bf16_nearest(v) for v in o], np.uint16)
    assert np.array_equal(r["logits"], lg)
    vals = [exact.bf16_exact(v) for v in lg]
    assert r["draft"] == vals.index(max(vals))
