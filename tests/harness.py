"""GPU-side helpers for the parity tests, the smoke check and the benchmark.

Uploads synthetic BF16 weights, runs the library through its Python binding,
and applies the comparison rules of the draft sweep:

  * FP8 codes and scales: bit-exact.
  * logits: max_v |g_v - o_v| <= tol_b, where g is the GPU's BF16 logit, o the
    oracle's unrounded FP64 logit and tol_b = 2e-2 * sigma_b (BF16 head) or
    6e-2 * sigma_b (FP8 head, against the FP8 oracle on the same bytes), sigma_b
    the population std of the oracle logits of sequence b.  When the BF16
    half-ulp at the largest |o| exceeds tol_b, BF16 storage alone could break
    the bound; the gate then widens to that half-ulp (and says so).
  * draft: equal to the oracle's whenever the oracle's top-1 / top-2 gap
    exceeds 2 tol_b; always equal to the lowest index of the GPU's own largest
    returned logit; always inside the oracle's near-max set {o_v >= o_max - 2 tol}.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import mtp_draft_head_embed_amd as mtp

TOL_BF16 = 2e-2
TOL_FP8 = 6e-2


def to_dev_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_order_key(b: np.ndarray) -> np.ndarray:
    """Integer key, monotone in the BF16 value, with +0 and -0 both 0; key
    differences count BF16 ulps."""
    b = np.asarray(b, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# Relative error of the library's FP32 norm value before its BF16 rounding:
# the sum of squares goes through at most 32 sequential fmaf per thread, a
# 6-level wave butterfly and at most 16 wave partials (all terms positive, so
# <= 54 roundings relative to the sum); the mean, + eps and the correctly
# rounded square root add 3, and the root halves the relative error: r is
# within 30 units (2^-24) of its exact value; the product x_j w_j is exact,
# and the library multiplies it by 1/r (one rounding for the reciprocal, one
# for the product): within 32 units.  64 units leaves a margin.
NORM_REL_ERR = 64 * 2.0 ** -24


def _bf16_from_key(k) -> np.ndarray:
    """Inverse of bf16_order_key (key 0 -> +0)."""
    k = np.asarray(k, dtype=np.int64)
    return np.where(k < 0, 0x8000 | (-k), k).astype(np.uint16)


def concat_flip_delta(concat: np.ndarray, concat_un: np.ndarray) -> np.ndarray:
    """Per concat entry, how far the library's BF16 value may lie from the
    oracle's: |c_other - c| where the unrounded oracle value u lies within
    NORM_REL_ERR |u| of the rounding boundary between c = BF16(u) and its
    neighbour c_other on u's side, else 0 (the library's FP32 norm value is
    then on the same side of every boundary, so it rounds to c exactly)."""
    c = bits_to_f64(concat)
    u = np.asarray(concat_un, dtype=np.float64)
    key = bf16_order_key(concat)
    other = np.where(u >= c, bits_to_f64(_bf16_from_key(key + 1)),
                     bits_to_f64(_bf16_from_key(key - 1)))
    mid = 0.5 * (c + other)
    slack = NORM_REL_ERR * np.abs(u) + 2.0 ** -149
    return np.where(np.abs(mid - u) <= slack, np.abs(other - c), 0.0)


def gpu_sum_depth(K: int) -> int:
    """Most FP32 roundings any product goes through in the library's sums of
    K terms: the row GEMV sums K/64 products per lane and 7 levels across the
    wave; an MFMA instruction adds 32 products to its accumulator (at most 32
    roundings, in whatever order), then one instruction per 32 columns of a
    K split, then at most 32 split partials in order."""
    return K // 32 + 64


def check_eh_proj_rows(xg: np.ndarray, x_un: np.ndarray, concat: np.ndarray,
                       concat_un: np.ndarray, eh_proj: np.ndarray) -> dict:
    """Compare BF16 eh_proj outputs from the library (bits [T][H]) with the
    oracle's unrounded FP64 values for the same rows.

    Every element: |g - o| <= ulp(max(|g|, |o|)) / 2 + D 2^-23 m' + f, where
      * c is the oracle's BF16 concat and f = sum_k |W_ik| d_k, d_k the most the
        library's BF16 concat entry can differ from c_k (concat_flip_delta:
        nonzero only for the few entries whose unrounded value lies within the
        FP32 norm's error of a BF16 rounding boundary);
      * m' = sum_k |W_ik| |c_k| + f bounds the sum of |products| the library
        adds, D = gpu_sum_depth(K) the roundings any of them goes through, and
        2^-23 one rounding (round-to-nearest or not);
      * the first term is the final BF16 rounding.
    Rows that nearly cancel (|o| << m') are held to the m'-scaled terms.

    Then the share of elements not bit-equal to the oracle's BF16 x, per row:
    under half of any row (rows of 256 or more), 1% of the median row, and at
    most 0.5% of the median row more than one ulp away.  Returns the
    statistics, including the median bound in ulps of |x|."""
    g = bits_to_f64(xg)
    o = np.asarray(x_un, dtype=np.float64)
    K = concat.shape[-1]

    def bf16_ulp(v):
        ex = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -133)))
        return 2.0 ** (np.maximum(ex, -126.0) - 7)

    cf = bits_to_f64(concat)
    absw = np.abs(bits_to_f64(eh_proj))
    flips = concat_flip_delta(concat, concat_un) @ absw.T
    m = np.abs(cf) @ absw.T + flips
    ulp = bf16_ulp(np.maximum(np.abs(g), np.abs(o)))
    bound = 0.5 * ulp + gpu_sum_depth(K) * 2.0 ** -23 * m + flips
    err = np.abs(g - o)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (worst, err[worst], bound[worst], o[worst], m[worst])
    from oracle import bf16_from_f64  # only the rounding of the oracle's own value
    d = np.abs(bf16_order_key(xg) - bf16_order_key(bf16_from_f64(o)))
    d = d.reshape(-1, d.shape[-1])
    ne_row = np.mean(d != 0, axis=1)
    over_row = np.mean(d > 1, axis=1)
    stats = {"elements": int(d.size), "not_equal": float(np.mean(d != 0)),
             "max_row_not_equal": float(ne_row.max()),
             "median_row_not_equal": float(np.median(ne_row)),
             "median_row_over_1ulp": float(np.median(over_row)), "max_ulps": int(d.max()),
             "median_bound_ulps": float(np.median(bound / bf16_ulp(o)))}
    if d.shape[1] >= 256:  # in shorter rows one flipped term can move most elements
        assert stats["max_row_not_equal"] < 0.5, stats
    assert stats["median_row_not_equal"] < 0.01, stats
    assert stats["median_row_over_1ulp"] < 0.005, stats
    return stats


@dataclasses.dataclass
class DevWeights:
    w: mtp.mtp_weights
    tensors: dict
    hidden: int
    vocab: int


def upload(weights: dict, device="cuda", with_lm_head=True) -> DevWeights:
    t = {k: to_dev_bf16(weights[k], device) for k in
         ("embed", "enorm_w", "hnorm_w", "head_norm_w", "eh_proj")}
    t["lm_head"] = to_dev_bf16(weights["lm_head"], device) if with_lm_head else None
    w = mtp.mtp_weights(t["embed"], t["enorm_w"], t["hnorm_w"], t["head_norm_w"], t["eh_proj"],
                        t["lm_head"], weights["rms_eps"])
    V, H = weights["embed"].shape
    return DevWeights(w, t, H, V)


def quantize_dev(dw: DevWeights, device="cuda"):
    V, H = dw.vocab, dw.hidden
    q = torch.empty((V, H), dtype=torch.uint8, device=device)
    s = torch.empty(V, dtype=torch.float32, device=device)
    ws = torch.empty(256, dtype=torch.uint8, device=device)
    mtp.mtp_quantize_head_fp8(dw.tensors["lm_head"], V, H, q, s, ws)
    return q, s


def run_draft(dw: DevWeights, tokens: np.ndarray, hidden: np.ndarray, fp8=None,
              with_logits=True, device="cuda"):
    """Returns (draft uint32 [B], logits BF16 bits [B][V] or None)."""
    B = int(tokens.size)
    tk = torch.from_numpy(tokens.astype(np.uint32).view(np.int32)).to(device)
    hd = to_dev_bf16(hidden.reshape(B, dw.hidden), device)
    dr = torch.empty(B, dtype=torch.int32, device=device)
    # NaN-filled, so a logit the call leaves unwritten fails every comparison
    lg = (torch.full((B, dw.vocab), float("nan"), dtype=torch.bfloat16, device=device)
          if with_logits else None)
    ws = mtp.new_workspace(dw.hidden, dw.vocab, B, device)
    if fp8 is None:
        mtp.mtp_draft_bf16(dw.w, B, tk, hd, dr, lg, ws)
    else:
        mtp.mtp_draft_fp8w(dw.w, fp8[0], fp8[1], B, tk, hd, dr, lg, ws)
    torch.cuda.synchronize()
    d = dr.cpu().numpy().view(np.uint32)
    return d, (bf16_bits(lg) if lg is not None else None)


@dataclasses.dataclass
class SeqReport:
    b: int
    sigma: float
    tol: float
    gate: float
    widened: bool
    max_err: float
    gap: float
    draft_gpu: int
    draft_oracle: int
    gated_exact: bool
    ok: bool
    why: str


def compare_sequence(b: int, o: np.ndarray, g_bits: np.ndarray | None, draft_gpu: int,
                     draft_oracle: int, tol_rel: float) -> SeqReport:
    """Apply the comparison rules to one sequence."""
    sigma = float(np.std(o))
    tol = tol_rel * sigma
    omax = float(np.max(np.abs(o)))
    # half-ulp of BF16 at the largest logit magnitude
    e = int(np.floor(np.log2(omax))) if omax > 0 else -126
    half_ulp = 2.0 ** (e - 8)
    gate = max(tol, half_ulp + 1e-6 * max(omax, 1.0))
    widened = gate > tol
    order = np.argsort(-o, kind="stable")
    top1 = float(o[order[0]])
    top2 = float(o[order[1]]) if o.size > 1 else -np.inf
    gap = top1 - top2
    why = []
    max_err = float("nan")
    if g_bits is not None:
        g = bits_to_f64(g_bits)
        max_err = float(np.max(np.abs(g - o)))
        if not max_err <= gate:
            why.append(f"logit error {max_err:.4g} > gate {gate:.4g}")
        m = g.max()
        own = int(np.nonzero(g == m)[0][0])
        if draft_gpu != own:
            why.append(f"draft {draft_gpu} is not the lowest argmax {own} of the returned logits")
    gated = gap > 2 * gate
    if gated and draft_gpu != draft_oracle:
        why.append(f"gap {gap:.4g} > 2 gate but draft {draft_gpu} != oracle {draft_oracle}")
    if not (0 <= draft_gpu < o.size) or o[draft_gpu] < top1 - 2 * gate:
        why.append(f"draft {draft_gpu} outside the near-max set")
    return SeqReport(b, sigma, tol, gate, widened, max_err, gap, int(draft_gpu), int(draft_oracle),
                     gated, not why, "; ".join(why))
