"""Near-tie stress construction (test helper; uses the oracle).

For each sequence b the oracle's normed activation xn_b is computed, and 64
lm_head rows P_b (disjoint across sequences) are overwritten so that their
logits lie within 1e-3 of a value c_b that sits 0.25 above the background
maximum: 16 rows are bit-identical copies of a base row r_b with
r_b . xn_b ~= c_b, and 48 are copies with one element moved by one BF16 ulp.
All planted logits of b then round to the same BF16 value c_b, so the lowest
planted index must win the argmax on the BF16 head -- a test of the argmax's
tie rule across workgroups and tiles.  The ids include 0, V-1, multiples of
64/256/1024 and their neighbours (tile and workgroup edges) and the last eighth
of the vocabulary; each sequence's lowest planted id sits in a different part
of the vocabulary.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import synth

N_PLANT = 64
N_COPIES = 16


@dataclasses.dataclass
class NearTie:
    lm_head: np.ndarray          # BF16 bits [V][H] with the planted rows
    planted: list                # per sequence: sorted planted ids
    c: list                      # per sequence: the BF16 value planted logits round to
    xn: list                     # per sequence: oracle xn (BF16 bits)


def _bf16_ceil(v: float) -> int:
    """Bits of the smallest BF16 value >= v (v > 0)."""
    b = int(oracle.bf16_from_f64(np.array([v]))[0])
    if oracle.bf16_to_f64(np.array([b], np.uint16))[0] < v:
        b += 1
    return b


def _ulp_step(bits: int, up: bool) -> int:
    """Neighbouring BF16 pattern (towards +inf when up)."""
    neg = bits & 0x8000
    mag = bits & 0x7FFF
    if mag == 0:
        return 0x0001 if up else 0x8001
    if (not neg) == up:
        return bits + 1
    return bits - 1


def _choose_ids(rng, V: int, B: int) -> list:
    used = set()
    out = []
    for b in range(B):
        ids = set()
        # lowest planted id of this sequence: near a 1024 boundary in its own
        # part of the vocabulary (0 for the first sequence)
        if b == 0:
            lo = 0
        else:
            lo = (int((b + 0.5) * V / B) // 1024) * 1024 + (b % 3) - 1
            lo = min(max(lo, 1), V - N_PLANT - 1)
        while lo in used:
            lo += 1
        ids.add(lo)
        if b == 1 and (V - 1) not in used:
            ids.add(V - 1)
        cands = []
        for m in (64, 256, 1024):
            k = int(rng.integers(lo // m + 1, max(lo // m + 2, V // m)))
            for d in (-1, 0, 1):
                cands.append(k * m + d)
        cands += list(rng.integers(V - V // 8, V, size=8))
        for c in cands:
            c = int(c)
            if lo < c < V and c not in used:
                ids.add(c)
        while len(ids) < N_PLANT:
            c = int(rng.integers(lo + 1, V))
            if c not in used:
                ids.add(c)
        ids = sorted(ids)
        assert len(ids) == N_PLANT and ids[0] == lo
        used.update(ids)
        out.append(ids)
    return out


def build(cfg: synth.Config, wts: dict, tokens: np.ndarray, hidden: np.ndarray,
          nthreads: int | None = None) -> NearTie:
    V, H, B = cfg.vocab, cfg.hidden, cfg.batch
    rng = synth.planting_rng(cfg)
    L = wts["lm_head"].copy()
    ids = _choose_ids(rng, V, B)
    xns, cs = [], []
    for b in range(B):
        r = oracle.draft(wts, int(tokens[b]), hidden[b], nthreads=nthreads)
        xn = r["xn"]
        xf = oracle.bf16_to_f64(xn)
        m_b = float(np.max(r["o"]))
        c_bits = _bf16_ceil(m_b + 0.25)
        c = float(oracle.bf16_to_f64(np.array([c_bits], np.uint16))[0])
        assert c < 16.0, "planted logit must stay below 16 (BF16 half-ulp <= tolerance)"
        base = oracle.bf16_from_f64(c * xf / float(np.dot(xf, xf)))
        rv = oracle.bf16_to_f64(base)
        o = float(np.dot(rv, xf))
        order = np.argsort(-np.abs(xf), kind="stable")
        for j in order:
            if abs(o - c) <= 1e-4:
                break
            if xf[j] == 0.0:
                continue
            up = (o < c) == (xf[j] > 0)
            nb = _ulp_step(int(base[j]), up)
            nv = float(oracle.bf16_to_f64(np.array([nb], np.uint16))[0])
            o2 = o + (nv - rv[j]) * xf[j]
            if abs(o2 - c) < abs(o - c):
                base[j] = nb
                rv[j] = nv
                o = o2
        o_exact = float(oracle.gemv_bf16(base[None, :], xn, nthreads=1)[0])
        assert abs(o_exact - c) <= 1e-4, (b, o_exact, c)
        rows = []
        for k in range(N_PLANT):
            if k < N_COPIES:
                rows.append(base.copy())
                continue
            while True:
                j = int(rng.integers(0, H))
                row = base.copy()
                row[j] = _ulp_step(int(row[j]), bool(rng.integers(0, 2)))
                ov = float(oracle.gemv_bf16(row[None, :], xn, nthreads=1)[0])
                if abs(ov - c) <= 1e-3:
                    rows.append(row)
                    break
        perm = rng.permutation(N_PLANT)
        for k, v in enumerate(ids[b]):
            L[v] = rows[perm[k]]
        xns.append(xn)
        cs.append(c)
    return NearTie(L, ids, cs, xns)


def verify(nt: NearTie, wts: dict, tokens, hidden, nthreads=None) -> list:
    """Oracle check of the planted matrix; returns per-sequence oracle results."""
    w2 = dict(wts)
    w2["lm_head"] = nt.lm_head
    res = []
    for b in range(len(nt.planted)):
        r = oracle.draft(w2, int(tokens[b]), hidden[b], nthreads=nthreads)
        o = r["o"]
        P = np.array(nt.planted[b])
        c = nt.c[b]
        assert np.all(np.abs(o[P] - c) <= 1e-3 + 1e-9), b
        mask = np.ones(o.size, bool)
        mask[P] = False
        assert o[mask].max() <= c - 0.2, (b, o[mask].max(), c)
        assert np.all(r["logits"][P] == r["logits"][P[0]])
        assert r["draft"] == P.min(), (b, r["draft"], P.min())
        res.append(r)
    return res
