"""Plain float64 CPU oracle (test infrastructure only; see the package docstring).

Parity pins for every function here live in ``tests/test_oracle_pins.py``.

Sources (pages as titled; section names as they appear there):
- "Continuous Decode Batching - the transformer capture": the decode step
  ("decode_step_batch - paint-by-numbers": per-sequence slab, RoPE at t_s,
  append at t_s, keys [0..=t_s], lm_head per token, then t_s += 1) and the
  segmented prefill ("REVISED: the hard kernel already exists": K segments in
  one pass, segment-local causal attention, no cross-segment leakage).
- mlx-bun "Batching" design note, section 5 ("per-sequence position"): one
  position per row, captured once per step and used for both Q and K.
- mlx-bun "Batching" design note (later revision), section 8: greedy argmax
  selects the lowest vocabulary id among tied scores.

Readings where the pages are silent (the pages never spell out the decoder
body; the plainest Llama/Mistral reading is taken):
- RMSNorm: y = x / sqrt(mean(x^2) + eps) * g.
- RoPE: rotate-half pairing (i, i + Dh/2), angle t * theta^(-2i/Dh), no scaling.
- GQA: query head h reads kv head floor(h / (Hq/Hkv)); scores scaled by 1/sqrt(Dh).
- SwiGLU FFN: W_down (silu(W_gate b) * (W_up b)), silu(z) = z / (1 + e^-z).
- Storage: K and V are rounded to bf16 (nearest-even) when written to a slab
  and attention reads the rounded values, so a prefill and the same tokens
  fed one at a time through decode attend to identical keys.
- int4 affine weights: w = scale * code + bias per group of consecutive
  input-dimension elements.
- Quantized K/V (``kv_format="affine8"`` or ``"affine4"``, module ``kvquant``):
  the slab keeps the affine 8-bit or 4-bit form of the bf16 value above,
  written when the token is appended; attention reads its dequantized value.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from .kvquant import dequantize_affine8, quantize_affine


# --------------------------------------------------------------------------- number formats

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, in one step.

    bf16 keeps 8 significant bits. Writing |x| = m * 2^e with 0.5 <= m < 1,
    the bf16 neighbours are multiples of 2^(e-8), so the result is
    rint(m * 2^8) * 2^(e-8) (numpy's rint rounds half to even). Values below
    the bf16 normal range are not expected here and are not treated
    specially."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def f64_to_bf16_bits(x) -> np.ndarray:
    """bf16 bit pattern of float64 values (rounded with :func:`round_to_bf16`)."""
    r = round_to_bf16(x).astype(np.float32)  # exact: bf16 values are fp32 values
    return (r.view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------- building blocks

def rmsnorm(x, g, eps: float) -> np.ndarray:
    """RMS normalisation over the last axis with gain g."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def rope_angles(position: int, head_dim: int, theta: float) -> np.ndarray:
    """Rotation angles of the Dh/2 pairs at one position: t * theta^(-2i/Dh)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / head_dim)
    return float(position) * inv_freq


def apply_rope(x, position: int, theta: float) -> np.ndarray:
    """Rotate every head vector in x[..., Dh] to position t (rotate-half pairing).

    Pair i is (x[i], x[i + Dh/2]); it is rotated by angle a_i:
    (x1, x2) -> (x1 cos a - x2 sin a, x2 cos a + x1 sin a)."""
    x = np.asarray(x, dtype=np.float64)
    dh = x.shape[-1]
    a = rope_angles(position, dh, theta)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : dh // 2], x[..., dh // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attend_one_head(q, keys, values) -> np.ndarray:
    """softmax(q . K^T / sqrt(Dh)) V for one query vector over all given keys."""
    q = np.asarray(q, dtype=np.float64)
    scores = keys @ q / np.sqrt(q.shape[-1])
    m = np.max(scores)
    p = np.exp(scores - m)
    p = p / np.sum(p)
    return p @ values


def silu(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def dequant_int4(codes, scale_bits, bias_bits, group: int) -> np.ndarray:
    """w[n, k] = scale[n, k // group] * code[n, k] + bias[n, k // group] (float64)."""
    codes = np.asarray(codes)
    s = np.repeat(bf16_bits_to_f64(scale_bits), group, axis=1)
    b = np.repeat(bf16_bits_to_f64(bias_bits), group, axis=1)
    return s * codes.astype(np.float64) + b


def greedy(logits) -> np.ndarray:
    """Per-row argmax; among equal maxima the lowest vocabulary id wins."""
    logits = np.atleast_2d(np.asarray(logits))
    out = np.empty(logits.shape[0], dtype=np.int64)
    for r in range(logits.shape[0]):
        row = logits[r]
        best = 0
        for v in range(1, row.shape[0]):
            if row[v] > row[best]:
                best = v
        out[r] = best
    return out


# --------------------------------------------------------------------------- sequence state

@dataclass
class SeqState:
    """One sequence's persistent slab: per-layer K and V, [len, Hkv, Dh] bf16 bits, or for affine8
    storage uint8 codes with (scale, bias) pairs in k_sb / v_sb ([len, Hkv, Dh/group, 2] float32)."""
    k: List[np.ndarray]
    v: List[np.ndarray]
    k_sb: Optional[List[np.ndarray]] = None
    v_sb: Optional[List[np.ndarray]] = None

    @property
    def length(self) -> int:
        return int(self.k[0].shape[0])


# --------------------------------------------------------------------------- the model

class OracleModel:
    """Random-init decoder evaluated row by row in float64.

    ``weights`` is the dict produced by ``synth.make_weights`` (bf16 bit
    patterns, or int4 dicts with ``codes``/``scale``/``bias``)."""

    def __init__(self, weights: Dict, cache_all_layers: bool = False, kv_format: str = "bf16",
                 kv_group: int = 64):
        if kv_format not in ("bf16", "affine8", "affine4"):
            raise ValueError("kv_format must be 'bf16', 'affine8' or 'affine4'")
        self.w = weights
        self.cfg = weights["shape"]
        self.kv_format = kv_format
        self.kv_group = kv_group
        self.seqs: Dict[int, SeqState] = {}
        self._next_id = 0
        self._cache: Dict = {}
        self._cache_all = cache_all_layers
        # Optional input: a callable (sid, layer, position, which, y, stored) -> stored, consulted for
        # every K ("k") or V ("v") vector the model computes itself before it enters the slab; y is
        # the unrounded float64 value [Hkv, Dh] and stored the slab form the model made of it (bf16
        # bits [1, Hkv, Dh], or (codes, pairs) for affine slabs). What it returns is stored instead:
        # a slab snapshot given as input. None: the model's own form.
        self.stored_override = None

    # -- weights
    def _matrix(self, m) -> np.ndarray:
        if isinstance(m, dict):
            return dequant_int4(m["codes"], m["scale"], m["bias"], self.cfg.group_size)
        return bf16_bits_to_f64(m)

    def dense(self, layer: int, name: str) -> np.ndarray:
        key = (layer, name)
        if key not in self._cache:
            if not self._cache_all:
                self._cache = {k: v for k, v in self._cache.items() if k[0] == layer}
            src = self.w[name] if layer < 0 else self.w["layers"][layer][name]
            self._cache[key] = self._matrix(src) if name not in ("attn_norm", "ffn_norm", "final_norm") \
                else bf16_bits_to_f64(src)
        return self._cache[key]

    def embed_rows(self, tokens) -> np.ndarray:
        return bf16_bits_to_f64(self.w["embed"][np.asarray(tokens, dtype=np.int64)])

    # -- sequences
    def new_sequence(self) -> int:
        c = self.cfg
        sid = self._next_id
        self._next_id += 1
        if self.kv_format == "bf16":
            empty = lambda: np.zeros((0, c.n_kv_heads, c.head_dim), dtype=np.uint16)
            self.seqs[sid] = SeqState([empty() for _ in range(c.n_layers)], [empty() for _ in range(c.n_layers)])
        else:
            ec = lambda: np.zeros((0, c.n_kv_heads, c.head_dim), dtype=np.uint8)
            es = lambda: np.zeros((0, c.n_kv_heads, c.head_dim // self.kv_group, 2), dtype=np.float32)
            L = range(c.n_layers)
            self.seqs[sid] = SeqState([ec() for _ in L], [ec() for _ in L], [es() for _ in L], [es() for _ in L])
        return sid

    def free_sequence(self, sid: int) -> None:
        del self.seqs[sid]

    def fork(self, parent: int, prefix_len: int) -> int:
        """A new sequence whose first prefix_len positions hold the parent's K/V (mlx-bun "Batching"
        design note, section 6 "KV memory model", item 3: block-level copy-on-write sharing of a prefix).
        Earlier positions never change once written (a slab only grows), so sharing them and copying
        them give the same values; the new sequence continues from position prefix_len."""
        p = self.seqs[parent]
        if not 0 <= prefix_len <= p.length:
            raise ValueError("prefix of %d tokens outside the parent's %d" % (prefix_len, p.length))
        sid = self.new_sequence()
        s = self.seqs[sid]
        for l in range(self.cfg.n_layers):
            s.k[l] = p.k[l][:prefix_len].copy()
            s.v[l] = p.v[l][:prefix_len].copy()
            if s.k_sb is not None:
                s.k_sb[l] = p.k_sb[l][:prefix_len].copy()
                s.v_sb[l] = p.v_sb[l][:prefix_len].copy()
        return sid

    def append_history(self, sid: int, k_bits, v_bits) -> None:
        """Append given K/V (bf16 bits, [L, n, Hkv, Dh]) to a slab."""
        for l in range(self.cfg.n_layers):
            self._store(self.seqs[sid], l, np.asarray(k_bits[l], dtype=np.uint16), np.asarray(v_bits[l], dtype=np.uint16))

    def _encode(self, bits: np.ndarray):
        """Slab form of bf16 K or V bits [n, Hkv, Dh]: the bits themselves, or affine (codes, pairs)."""
        if self.kv_format == "bf16":
            return bits
        return quantize_affine(bits, self.kv_group, 8 if self.kv_format == "affine8" else 4)

    def _put(self, s: SeqState, l: int, which: str, stored) -> None:
        """Append a slab form made by _encode to layer l of K ("k") or V ("v")."""
        if self.kv_format == "bf16":
            arr = s.k if which == "k" else s.v
            arr[l] = np.concatenate([arr[l], stored])
            return
        codes, sbs = (s.k, s.k_sb) if which == "k" else (s.v, s.v_sb)
        codes[l] = np.concatenate([codes[l], stored[0]])
        sbs[l] = np.concatenate([sbs[l], stored[1]])

    def _store(self, s: SeqState, l: int, kb: np.ndarray, vb: np.ndarray) -> None:
        """Append bf16 K/V bits [n, Hkv, Dh] to layer l of a slab, in the slab's storage format."""
        self._put(s, l, "k", self._encode(kb))
        self._put(s, l, "v", self._encode(vb))

    def kv_values(self, sid: int, l: int):
        """Values attention reads from layer l of a slab: (K, V) float64 [len, Hkv, Dh]."""
        s = self.seqs[sid]
        if self.kv_format == "bf16":
            return bf16_bits_to_f64(s.k[l]), bf16_bits_to_f64(s.v[l])
        return (dequantize_affine8(s.k[l], s.k_sb[l], self.kv_group),
                dequantize_affine8(s.v[l], s.v_sb[l], self.kv_group))

    def copy_state(self) -> Dict[int, SeqState]:
        cp = lambda xs: None if xs is None else [a.copy() for a in xs]
        return {sid: SeqState(cp(s.k), cp(s.v), cp(s.k_sb), cp(s.v_sb)) for sid, s in self.seqs.items()}

    # -- one layer for a set of (row, position) queries
    def _layer(self, l: int, h: np.ndarray, rows: Sequence[int], positions: Sequence[int]) -> np.ndarray:
        """Apply decoder layer l to hidden rows h[i] of sequence rows[i] at positions[i].

        Each query i writes its K/V at positions[i] of its own slab, then
        attends to keys [0..=positions[i]] of that slab only. Queries of one
        sequence must be listed in increasing position order and the slab
        must already hold every earlier position."""
        c = self.cfg
        g = c.n_heads // c.n_kv_heads
        a = rmsnorm(h, self.dense(l, "attn_norm"), c.rms_eps)
        q = (a @ self.dense(l, "wq").T).reshape(len(rows), c.n_heads, c.head_dim)
        k = (a @ self.dense(l, "wk").T).reshape(len(rows), c.n_kv_heads, c.head_dim)
        v = (a @ self.dense(l, "wv").T).reshape(len(rows), c.n_kv_heads, c.head_dim)
        # K/V of every query first (causal, so a later write is never read early)
        for i, (sid, t) in enumerate(zip(rows, positions)):
            s = self.seqs[sid]
            if s.k[l].shape[0] != t:
                raise ValueError("slab length %d != position %d" % (s.k[l].shape[0], t))
            for which, y in (("k", apply_rope(k[i], t, c.rope_theta)), ("v", v[i])):
                stored = self._encode(f64_to_bf16_bits(y)[None])
                if self.stored_override is not None:
                    stored = self.stored_override(sid, l, t, which, y, stored)
                self._put(s, l, which, stored)
        o = np.zeros((len(rows), c.n_heads, c.head_dim))
        kv_f64 = {}
        for i, (sid, t) in enumerate(zip(rows, positions)):
            if sid not in kv_f64:  # one sequence's values at a time (a long slab is large in float64)
                kv_f64 = {sid: self.kv_values(sid, l)}
            K, V = kv_f64[sid]
            qr = apply_rope(q[i], t, c.rope_theta)
            for hh in range(c.n_heads):
                j = hh // g
                o[i, hh] = attend_one_head(qr[hh], K[: t + 1, j], V[: t + 1, j])
        h = h + o.reshape(len(rows), -1) @ self.dense(l, "wo").T
        b = rmsnorm(h, self.dense(l, "ffn_norm"), c.rms_eps)
        m = silu(b @ self.dense(l, "w_gate").T) * (b @ self.dense(l, "w_up").T)
        return h + m @ self.dense(l, "w_down").T

    def _head(self, h: np.ndarray) -> np.ndarray:
        x = rmsnorm(h, self.dense(-1, "final_norm"), self.cfg.rms_eps)
        return x @ self.dense(-1, "lm_head").T

    # -- the two entry points
    def decode_step_batch(self, seq_ids: Sequence[int], last_tokens: Sequence[int]) -> np.ndarray:
        """One decode step for B distinct live sequences; returns logits [B, V].

        Row i uses t = its slab length, writes its K/V at t, attends [0..=t],
        and its length becomes t + 1."""
        seq_ids = [int(s) for s in seq_ids]
        if len(set(seq_ids)) != len(seq_ids):
            raise ValueError("duplicate sequence id in one step")
        if not seq_ids:
            return np.zeros((0, self.cfg.vocab))
        positions = [self.seqs[s].length for s in seq_ids]
        h = self.embed_rows(last_tokens)
        for l in range(self.cfg.n_layers):
            h = self._layer(l, h, seq_ids, positions)
        return self._head(h)

    def prefill(self, sid: int, tokens) -> np.ndarray:
        """Causal forward of one sequence's tokens from its current length; logits of the last token."""
        tokens = np.asarray(tokens, dtype=np.int64)
        if tokens.size == 0:
            raise ValueError("empty segment")
        t0 = self.seqs[sid].length
        positions = list(range(t0, t0 + tokens.size))
        h = self.embed_rows(tokens)
        for l in range(self.cfg.n_layers):
            h = self._layer(l, h, [sid] * tokens.size, positions)
        return self._head(h[-1:])[0]

    def prefill_segmented(self, seq_ids: Sequence[int], segments: Sequence) -> np.ndarray:
        """K segments, each its own causal forward (no cross-segment attention); logits [K, V]."""
        if len(set(int(s) for s in seq_ids)) != len(seq_ids):
            raise ValueError("duplicate sequence id in one prefill")
        out = [self.prefill(int(s), seg) for s, seg in zip(seq_ids, segments)]
        return np.stack(out) if out else np.zeros((0, self.cfg.vocab))
