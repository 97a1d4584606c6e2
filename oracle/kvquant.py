"""Plain CPU definition of affine 8-bit and 4-bit K/V storage (test infrastructure only; see the package
docstring).

Sources (pages as titled; section names as they appear there):
- mlx-bun "Batching" design note, section 4.3 "Join: adopt, extend, or merge - by layer kind": a
  quantized full-attention cache is held as (packed values, scales, biases) triples.
- The same note, section 6 "KV memory model": quantized K/V multiplies the capacity of the budget.
- mlx-bun "Batching perf path" note, section 2 "Gap analysis: quantized KV at B>1": the quantized
  cache is the same per-row state as the bf16 one, attended through dequantization.
- mlx-bun "Batching" design note (later revision), section 8 "Open items", "Consolidation matrix":
  affine K/V in 8-bit and 4-bit forms (KV8, KV4) made of packed values, scales and biases.

Readings where the pages are silent (the plainest ones, listed in the design notes):
- Affine groups of 64 consecutive elements of one head vector (the head dimension), one group
  per 64 dims; each group stores a scale s and a bias b, and an element is s * code + b.
- Quantized value x is the bf16 value that a bf16 slab would hold for that element.
- b = the group minimum, s = (group maximum - b) / L, code = round-half-even((x - b) / s)
  clamped to 0..L, and code 0 for a constant group (s = 0), with L = 255 (8-bit) or 15 (4-bit).
  The code is an integer decided by floating point, so it is decided in float32, the storage
  precision of s and b: the subtraction and the division are single float32 operations (IEEE,
  rounded to nearest).
- Dequantized values (what attention reads) are s * code + b evaluated exactly (float64).
"""
from __future__ import annotations

import numpy as np

KV8_LEVELS = 255


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantize_affine8(bits, group: int = 64):
    """bf16 bit patterns [..., D] -> (codes uint8 [..., D], sb float32 [..., D/group, 2] = (scale, bias))."""
    return quantize_affine(bits, group, 8)


def quantize_affine4(bits, group: int = 64):
    """The 4-bit form: codes 0..15 (one per uint8 here), the same (scale, bias) pairs."""
    return quantize_affine(bits, group, 4)


def quantize_affine(bits, group: int = 64, nbits: int = 8):
    """Affine codes of nbits bits per element with a (scale, bias) pair per group."""
    levels = (1 << nbits) - 1
    x = bf16_bits_to_f32(bits)
    d = x.shape[-1]
    if d % group:
        raise ValueError("head dim %d is not a multiple of the group %d" % (d, group))
    xg = x.reshape(x.shape[:-1] + (d // group, group))
    lo = xg.min(axis=-1)
    hi = xg.max(axis=-1)
    scale = (hi - lo) / np.float32(levels)  # float32 operations throughout
    safe = np.where(scale > 0, scale, np.float32(1))
    q = np.rint((xg - lo[..., None]) / safe[..., None])
    q = np.where(scale[..., None] > 0, np.clip(q, 0, levels), 0)
    codes = q.astype(np.uint8).reshape(x.shape)
    sb = np.stack([scale, lo], axis=-1).astype(np.float32)
    return codes, sb


def dequantize_affine8(codes, sb, group: int = 64) -> np.ndarray:
    """x = scale * code + bias per group, exactly (float64)."""
    c = np.asarray(codes).astype(np.float64)
    sb = np.asarray(sb, dtype=np.float32).astype(np.float64)
    s = np.repeat(sb[..., 0], group, axis=-1)
    b = np.repeat(sb[..., 1], group, axis=-1)
    return s * c + b
