"""Seeded synthetic inputs for the MTP draft sweep.

This module only draws random numbers and stores them as BF16 bit patterns
(uint16, round to nearest even from float32).  It holds none of the sweep's
arithmetic.  Both the oracle-side tests and the HIP-side runs take their inputs
from here, so both see the same bytes.

Every tensor is drawn from ``numpy.random.Generator(PCG64(SeedSequence([seed,
tensor_id, chunk])))``, in fixed row chunks, so the bytes do not depend on how
many threads fill them.

No trained GLM-5.3 weights exist here; the shapes and value distributions stand
in for the draft head:
  weights (embed, eh_proj, lm_head) ~ N(0, 0.02); norm weights ~ 1 + N(0, 0.1);
  target hidden ~ N(0, 1) (Student-t with 3 degrees of freedom for the near-tie
  stress); tokens uniform in [0, vocab) (distinct when asked); rms_eps = 1e-6.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

TENSOR_IDS = {
    "embed": 0, "enorm_w": 1, "hnorm_w": 2, "eh_proj": 3, "head_norm_w": 4,
    "lm_head": 5, "hidden": 6, "tokens": 7, "planting": 8,
}


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    hidden: int
    vocab: int
    batch: int
    seed: int
    hidden_dist: str = "normal"     # "normal" or "t3"
    distinct_tokens: bool = False
    rms_eps: float = 1e-6


CONFIGS = {
    "tiny": Config("tiny", 256, 4096, 1, 1001),
    "mid": Config("mid", 4096, 151552, 1, 1002),
    "large": Config("large", 6144, 154880, 1, 1003),
    "batched": Config("batched", 6144, 154880, 16, 1004, distinct_tokens=True),
    "neartie": Config("neartie", 6144, 154880, 8, 1005, hidden_dist="t3",
                      distinct_tokens=True),
}


def rng(seed: int, tensor: str, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), TENSOR_IDS[tensor], int(chunk)])))


def to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def from_bf16(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(rows: int, cols: int, seed: int, tensor: str, mean: float, std: float,
                threads: int | None = None) -> np.ndarray:
    """[rows][cols] BF16 draws of N(mean, std), filled in fixed row chunks."""
    out = np.empty((rows, cols), dtype=np.uint16)
    per = max(1, (1 << 22) // max(1, cols))
    nchunks = (rows + per - 1) // per

    def fill(c):
        r0, r1 = c * per, min(rows, (c + 1) * per)
        a = rng(seed, tensor, c).standard_normal((r1 - r0, cols), dtype=np.float32)
        a *= np.float32(std)
        if mean != 0.0:
            a += np.float32(mean)
        out[r0:r1] = to_bf16(a)

    if nchunks == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def make_weights(cfg: Config, threads: int | None = None) -> dict:
    """BF16 head weights for a config: embed [V][H], eh_proj [H][2H],
    lm_head [V][H], enorm_w / hnorm_w / head_norm_w [H]."""
    H, V, s = cfg.hidden, cfg.vocab, cfg.seed
    return {
        "embed": normal_bf16(V, H, s, "embed", 0.0, 0.02, threads),
        "enorm_w": normal_bf16(1, H, s, "enorm_w", 1.0, 0.1)[0],
        "hnorm_w": normal_bf16(1, H, s, "hnorm_w", 1.0, 0.1)[0],
        "eh_proj": normal_bf16(H, 2 * H, s, "eh_proj", 0.0, 0.02, threads),
        "head_norm_w": normal_bf16(1, H, s, "head_norm_w", 1.0, 0.1)[0],
        "lm_head": normal_bf16(V, H, s, "lm_head", 0.0, 0.02, threads),
        "rms_eps": cfg.rms_eps,
        "hidden_size": H,
        "vocab": V,
    }


def make_inputs(cfg: Config) -> tuple[np.ndarray, np.ndarray]:
    """(tokens uint32 [B], hidden BF16 [B][H]) for a config."""
    B, H, V = cfg.batch, cfg.hidden, cfg.vocab
    g = rng(cfg.seed, "tokens")
    if cfg.distinct_tokens:
        tokens = g.choice(V, size=B, replace=False).astype(np.uint32)
    else:
        tokens = g.integers(0, V, size=B, dtype=np.int64).astype(np.uint32)
    gh = rng(cfg.seed, "hidden")
    if cfg.hidden_dist == "t3":
        h = gh.standard_t(3, size=(B, H)).astype(np.float32)
    else:
        h = gh.standard_normal((B, H), dtype=np.float32)
    return tokens, to_bf16(h)


def planting_rng(cfg: Config) -> np.random.Generator:
    """Random stream for the near-tie planting choices (ids, nudges)."""
    return rng(cfg.seed, "planting")


def custom(hidden: int, vocab: int, batch: int, seed: int, **kw) -> Config:
    """A config of arbitrary shape with the standard distributions."""
    return Config(f"h{hidden}_v{vocab}_b{batch}_s{seed}", hidden, vocab, batch, seed, **kw)
