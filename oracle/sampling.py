"""Plain CPU definition of seeded per-row sampling (test infrastructure only; see the package docstring).

Sources (pages as titled; section names as they appear there):
- mlx-bun "Batching" design note (later revision), section 4.4 "The decode step", the paragraph
  on the sampling boundary: a row's random draw is selected by the request's seed and its local
  sample index, independently of the other rows in the batch.
- The same section, the paragraph on vectorized homogeneous sampling: temperature 0 is plain
  greedy selection, with the greedy tie rule (the lowest id among tied scores, section 8).

Readings where the pages are silent (the plainest ones, listed in the design notes):
- Temperature T > 0 divides the logits; the distribution is their softmax.
- Top-p: tokens ordered by probability, highest first, equal probabilities by lower id first;
  the nucleus is the shortest prefix of that order whose mass reaches p (at least one token).
- One uniform draw u in [0, 1) per row and step: the first 64-bit word of the Philox4x64-10
  block (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011)
  with key (seed, 0) and counter (sample index, 0, 0, 0); u = (word >> 40) / 2^24, so u has 24
  bits and is exact in float32 and float64.
- The token is the first one of the nucleus order whose cumulative mass exceeds u times the
  nucleus mass (inverse CDF over the renormalised nucleus).
Arithmetic is float64; the draw is integer arithmetic.
"""
from __future__ import annotations

import numpy as np

_MASK64 = (1 << 64) - 1
# Philox4x64 round multipliers and key increments (Weyl constants) from the SC 2011 paper
_PHILOX_M0 = 0xD2E7470EE14C6C93
_PHILOX_M1 = 0xCA5A826395121157
_PHILOX_W0 = 0x9E3779B97F4A7C15
_PHILOX_W1 = 0xBB67AE8584CAA73B


def philox4x64_10(counter, key):
    """Philox4x64 with 10 rounds: counter (4 x uint64), key (2 x uint64) -> 4 x uint64.

    A round multiplies words 0 and 2 by the two multipliers (128-bit products), then the new words
    are (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)); the key is bumped by the
    Weyl constants between rounds."""
    c = [int(x) & _MASK64 for x in counter]
    k = [int(x) & _MASK64 for x in key]
    for _ in range(10):
        p0 = c[0] * _PHILOX_M0
        p1 = c[2] * _PHILOX_M1
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & _MASK64, (p0 >> 64) ^ c[3] ^ k[1], p0 & _MASK64]
        k = [(k[0] + _PHILOX_W0) & _MASK64, (k[1] + _PHILOX_W1) & _MASK64]
    return c


def uniform_draw(seed: int, index: int) -> float:
    """The row's draw u in [0, 1): 24 high bits of Philox word 0 for key (seed, 0), counter (index, 0, 0, 0)."""
    w = philox4x64_10([index, 0, 0, 0], [seed, 0])[0]
    return float(w >> 40) / float(1 << 24)


def nucleus_order(logits, temperature: float, top_p: float):
    """(order, probabilities, cumulative, nucleus size) for one row; temperature > 0, 0 < top_p <= 1."""
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    e = np.exp(z - np.max(z))
    p = e / np.sum(e)
    ids = np.arange(p.shape[0])
    order = np.lexsort((ids, -p))  # probability descending, then id ascending
    cum = np.cumsum(p[order])
    n = int(np.searchsorted(cum, top_p, side="left")) + 1  # shortest prefix with mass >= top_p
    return order, p, cum, min(n, p.shape[0])


def sample_row(logits, temperature: float, top_p: float, seed: int, index: int) -> int:
    """One row's token: greedy at temperature 0, else top-p sampling with the seeded draw."""
    logits = np.asarray(logits, dtype=np.float64)
    if temperature == 0:
        best = 0
        for v in range(1, logits.shape[0]):
            if logits[v] > logits[best]:
                best = v
        return best
    order, p, cum, n = nucleus_order(logits, temperature, top_p)
    t = uniform_draw(seed, index) * cum[n - 1]
    j = int(np.searchsorted(cum[:n], t, side="right"))  # first cumulative mass above t
    return int(order[min(j, n - 1)])


def sample_rows(logits, temperature, top_p, seeds, indices) -> np.ndarray:
    logits = np.atleast_2d(np.asarray(logits))
    return np.array([sample_row(logits[r], float(temperature[r]), float(top_p[r]), int(seeds[r]), int(indices[r]))
                     for r in range(logits.shape[0])], dtype=np.int64)
