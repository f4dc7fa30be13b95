"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

This module only draws random numbers and names workload shapes.  It holds no
part of the layer's arithmetic (no sign handling, no decomposition, no
reconstruction, no product): the oracle and the HIP library each implement
that on their own, and both receive the arrays made here.

Conventions of the arrays produced:

* sign bits: ``uint8[m, d // 8]``, row-major, the least significant bit of a
  byte is the lowest column, and a set bit means the sign is -1.  Uniform
  random bytes give independent Bernoulli(0.5) signs.
* factors ``U`` (``m x k``) and ``V`` (``d x k``): ``float16``, row-major.
* activations ``x``: ``float16[M, d]``, row-major.

Every generator takes an integer seed plus a tuple of integers ("tags") that
identify the array (layer, weight, block ...), so any array can be regenerated
alone, in any order, with ``numpy.random.default_rng([seed, *tags])`` (PCG64).
"""
from __future__ import annotations

import numpy as np

# Decoder-layer linear shapes (name, out_features m, in_features d) of the two
# model families whose block sizes the pages discuss (Llama 3 8B; Llama 2 70B).
LLAMA3_8B_LAYER = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 14336, 4096),
    ("up", 14336, 4096),
    ("down", 4096, 14336),
)
LLAMA2_70B_LAYER = (
    ("q", 8192, 8192),
    ("k", 1024, 8192),
    ("v", 1024, 8192),
    ("o", 8192, 8192),
    ("gate", 28672, 8192),
    ("up", 28672, 8192),
    ("down", 8192, 28672),
)
LLAMA2_70B_LAYERS = 80

FACTOR_SCALE = 0.05  # U, V entries are |N(0, 1)| * 0.05 in the synthetic stacks
WEIGHT_STD = 0.02  # decomposed weight W ~ N(0, 0.02^2)


def rng(seed: int, *tags: int) -> np.random.Generator:
    """PCG64 generator for the array identified by (seed, *tags)."""
    return np.random.default_rng([int(seed), *[int(t) for t in tags]])


def gaussian_weight(seed: int, m: int, d: int, std: float = WEIGHT_STD) -> np.ndarray:
    """Dense fp32 weight ``W[m, d]`` with i.i.d. N(0, std^2) entries."""
    return (rng(seed, 1).standard_normal((m, d)) * std).astype(np.float32)


def sign_bits(seed: int, m: int, d: int, *tags: int) -> np.ndarray:
    """Uniform random packed sign bits ``uint8[m, d // 8]`` (Bernoulli(0.5) signs)."""
    if d % 8:
        raise ValueError("d must be a multiple of 8")
    g = rng(seed, 2, *tags)
    return np.frombuffer(g.bytes(m * (d // 8)), dtype=np.uint8).reshape(m, d // 8).copy()


def factor(seed: int, rows: int, k: int, *tags: int, scale: float = FACTOR_SCALE) -> np.ndarray:
    """fp16 factor ``[rows, k]`` with entries |N(0,1)| * scale (rounded to nearest even)."""
    g = rng(seed, 3, *tags)
    return (np.abs(g.standard_normal((rows, k))) * scale).astype(np.float16)


def dyadic_factor(seed: int, rows: int, k: int, *tags: int) -> np.ndarray:
    """fp16 factor ``[rows, k]`` whose entries are 1/4 or 1/2, each drawn with
    probability 1/2 (seeded per array, so every row, column and rank varies)."""
    g = rng(seed, 10, *tags)
    return np.where(g.integers(0, 2, size=(rows, k)) == 1, 0.5, 0.25).astype(np.float16)


def activations(seed: int, M: int, d: int, *tags: int) -> np.ndarray:
    """fp16 activations ``x[M, d]`` ~ N(0, 1)."""
    g = rng(seed, 4, *tags)
    return g.standard_normal((M, d)).astype(np.float16)


def synthetic_blocks(seed: int, m: int, d: int, n: int, k: int = 16, *tags: int):
    """``n`` synthetic residual blocks for one weight: list of dicts with keys
    ``bits`` (uint8[m, d/8]), ``u`` (fp16[m, k]) and ``v`` (fp16[d, k])."""
    out = []
    for i in range(n):
        out.append(
            {
                "bits": sign_bits(seed, m, d, *tags, i),
                "u": factor(seed, m, k, *tags, i, 0),
                "v": factor(seed, d, k, *tags, i, 1),
            }
        )
    return out


def block_counts(seed: int, count: int, lo: int, hi: int, *tags: int) -> np.ndarray:
    """Per-weight block counts drawn uniformly from the integers ``lo..hi``."""
    g = rng(seed, 5, *tags)
    return g.integers(lo, hi + 1, size=count).astype(np.int32)


def dyadic_blocks(seed: int, m: int, d: int, n: int, k: int = 16, *tags: int):
    """``n`` blocks with Bernoulli(0.5) sign bits and ``dyadic_factor`` U and V."""
    return [
        {
            "bits": sign_bits(seed, m, d, *tags, i),
            "u": dyadic_factor(seed, m, k, *tags, i, 0),
            "v": dyadic_factor(seed, d, k, *tags, i, 1),
        }
        for i in range(n)
    ]


def integer_activations(seed: int, M: int, d: int, lo: int = -2, hi: int = 2, *tags: int) -> np.ndarray:
    """fp16 activations drawn uniformly from the integers ``lo..hi``."""
    g = rng(seed, 6, *tags)
    return g.integers(lo, hi + 1, size=(M, d)).astype(np.float16)


def sample_rows(seed: int, m: int, count: int, *tags: int) -> np.ndarray:
    """Sorted distinct row indices, always including the first and last row."""
    g = rng(seed, 7, *tags)
    count = min(count, m)
    picked = set(g.choice(m, size=count, replace=False).tolist())
    picked.update({0, m - 1})
    return np.array(sorted(picked), dtype=np.int64)


def channel_magnitudes(seed: int, d: int, *tags: int, outlier_frac: float = 0.01) -> np.ndarray:
    """Positive per-input-channel activation magnitudes ``float32[d]``: log-normal
    exp(N(0, 0.5^2)), with a fraction ``outlier_frac`` of channels (at least one) made
    8 to 32 times larger, the outlier channels of LLM activations."""
    g = rng(seed, 8, *tags)
    mag = np.exp(0.5 * g.standard_normal(d))
    n_out = max(1, int(round(outlier_frac * d)))
    idx = g.choice(d, size=n_out, replace=False)
    mag[idx] *= g.uniform(8.0, 32.0, size=n_out)
    return mag.astype(np.float32)


def outlier_activations(seed: int, M: int, d: int, magnitudes: np.ndarray, *tags: int) -> np.ndarray:
    """fp16 activations ``x[M, d]``: N(0, 1) times the channel's magnitude."""
    g = rng(seed, 9, *tags)
    return (g.standard_normal((M, d)) * np.asarray(magnitudes, dtype=np.float64)[None, :]).astype(np.float16)


def inv_input_scale(seed: int, d: int, *tags: int) -> np.ndarray:
    """A positive per-input-channel factor ``float32[d]`` to fold into V: the reciprocal
    of ``channel_magnitudes(...) ** 0.5`` (a square-root damping of the channel
    magnitudes), so ordinary channels get factors near 1 and outlier channels ~1/3..1/6."""
    return (1.0 / np.sqrt(channel_magnitudes(seed, d, *tags).astype(np.float64))).astype(np.float32)
