"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module draws random tensors and nothing else: it holds none of the
decode method's arithmetic (no norm, projection, RoPE, attention or
sampling). Both sides of every parity check consume the arrays it returns.

Model shapes follow the workloads the pages' throughput argument is about:
a tiny decoder, a Llama-3-8B-shaped decoder and a Mistral-7B-shaped decoder
with 4-bit affine group-quantized weights. All models are random-init; the
pages' own systems ran trained checkpoints that are not reproduced here.

Conventions
- bf16 tensors are numpy ``uint16`` arrays holding the bf16 bit pattern.
- Matrices are ``[out_features, in_features]`` row-major (``y = W x``).
- Every tensor is drawn from its own counter-based stream, keyed by
  ``(seed, stream id)``, so any tensor (or any slice of one) can be
  regenerated independently and results do not depend on thread count.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "_gen.c")
_LIB_PATH = os.path.join(_HERE, "_synth_gen.so")
_lib = None


def build_generator(force: bool = False) -> str:
    """Compile the C generator (gcc, pthreads). Returns the .so path."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-Wall", "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build_generator())
        u64, i32, vp, f64 = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, f64, f64, vp, i32]
        lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, f64, f64, vp, i32]
        lib.synth_uniform_u32.argtypes = [u64, u64, u64, u64, u64, vp, i32]
        lib.synth_uniform_u8.argtypes = [u64, u64, u64, u64, u64, vp, i32]
        lib.synth_uniform_f64.argtypes = [u64, u64, u64, u64, vp, i32]
        for f in (lib.synth_normal_bf16, lib.synth_normal_f32, lib.synth_uniform_u32,
                  lib.synth_uniform_u8, lib.synth_uniform_f64):
            f.restype = None
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


# --------------------------------------------------------------------------- raw draws

def normal_bf16(seed: int, stream: int, shape, std: float = 1.0, mean: float = 0.0,
                offset: int = 0) -> np.ndarray:
    """bf16 bits of mean + std*N(0,1), elements ``offset .. offset+size`` of the stream."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().synth_normal_bf16(seed, stream, offset, n, mean, std, out.ctypes.data, _threads())
    return out.reshape(shape)


def normal_f32(seed: int, stream: int, shape, std: float = 1.0, mean: float = 0.0,
               offset: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    if n:
        _load().synth_normal_f32(seed, stream, offset, n, mean, std, out.ctypes.data, _threads())
    return out.reshape(shape)


def uniform_int(seed: int, stream: int, shape, n_range: int, offset: int = 0,
                dtype=np.uint32) -> np.ndarray:
    """Integers uniform in ``[0, n_range)`` (uint8 storage when ``dtype`` is uint8)."""
    n = int(np.prod(shape))
    if dtype == np.uint8:
        assert n_range <= 256
        out = np.empty(n, dtype=np.uint8)
        if n:
            _load().synth_uniform_u8(seed, stream, offset, n, n_range, out.ctypes.data, _threads())
    else:
        out = np.empty(n, dtype=np.uint32)
        if n:
            _load().synth_uniform_u32(seed, stream, offset, n, n_range, out.ctypes.data, _threads())
    return out.reshape(shape)


def uniform_f64(seed: int, stream: int, shape, offset: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float64)
    if n:
        _load().synth_uniform_f64(seed, stream, offset, n, out.ctypes.data, _threads())
    return out.reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest-even); returns the uint16 bit pattern."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- model shapes

@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rope_theta: float
    rms_eps: float = 1e-5
    weight_format: str = "bf16"      # "bf16" or "int4"
    group_size: int = 64             # int4 affine group along the input dim
    weight_std: float = 0.02

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def matrix_shapes(self) -> Dict[str, tuple]:
        d, f = self.d_model, self.ffn_dim
        return {"wq": (self.q_dim, d), "wk": (self.kv_dim, d), "wv": (self.kv_dim, d),
                "wo": (d, self.q_dim), "w_gate": (f, d), "w_up": (f, d), "w_down": (d, f)}

    def streamed_params(self) -> int:
        per_layer = sum(a * b for a, b in self.matrix_shapes().values())
        return self.n_layers * per_layer + self.vocab * self.d_model

    def kv_bytes_per_token(self) -> int:
        """bf16 K and V for one token across all layers."""
        return self.n_layers * 2 * self.kv_dim * 2


TINY = ModelShape("tiny", 2, 256, 4, 2, 64, 1024, 1024, 10000.0)
LLAMA8B = ModelShape("llama3-8b-shape", 32, 4096, 32, 8, 128, 14336, 128256, 500000.0)
# theta is not given for this shape; 1e6 is the value published with the
# Mistral-7B shape whose vocabulary is 32768 (a reading; it changes no bytes).
MISTRAL7B_INT4 = ModelShape("mistral7b-shape-int4", 32, 4096, 32, 8, 128, 14336, 32768, 1000000.0,
                            weight_format="int4")

SHAPES = {s.name: s for s in (TINY, LLAMA8B, MISTRAL7B_INT4)}

_MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
_NORMS = ("attn_norm", "ffn_norm")


def _stream_id(layer: int, name: str) -> int:
    names = _MATS + _NORMS + ("embed", "lm_head", "final_norm")
    return (layer + 1) * 1024 + names.index(name) * 8


BF16_ONE = np.uint16(0x3F80)


def _int4_matrix(seed: int, stream: int, shape, group: int, std: float) -> Dict[str, np.ndarray]:
    """Codes uniform 0..15; per-group scale = (std/4.61)*U(0.5,1.5) and bias = -7.5*scale, bf16.

    The dequantized weight scale*q + bias is then zero-mean with standard
    deviation close to ``std`` (the standard deviation of q-7.5 for q uniform
    on 0..15 is sqrt(255/12) = 4.61)."""
    n, k = shape
    assert k % group == 0
    codes = uniform_int(seed, stream, shape, 16, dtype=np.uint8)
    u = uniform_f64(seed, stream + 1, (n, k // group))
    scale_f = (std / 4.61) * (0.5 + u)
    scale = f32_to_bf16_bits(scale_f.astype(np.float32))
    bias = f32_to_bf16_bits((-7.5 * bf16_bits_to_f32(scale)).astype(np.float32))
    return {"codes": codes, "scale": scale, "bias": bias}


def make_weights(shape: ModelShape, seed: int, gain_std: float = 0.0,
                 layers: Optional[List[int]] = None) -> Dict:
    """Random-init weights: matrices and embeddings N(0, std^2) in bf16 (or int4-affine).

    Norm gains are exactly 1 unless ``gain_std`` > 0, in which case they are
    1 + N(0, gain_std^2) rounded to bf16."""
    d, v = shape.d_model, shape.vocab
    std = shape.weight_std
    w: Dict = {"shape": shape, "seed": seed}
    w["embed"] = normal_bf16(seed, _stream_id(-1, "embed"), (v, d), std)
    if shape.weight_format == "int4":
        w["lm_head"] = _int4_matrix(seed, _stream_id(-1, "lm_head"), (v, d), shape.group_size, std)
    else:
        w["lm_head"] = normal_bf16(seed, _stream_id(-1, "lm_head"), (v, d), std)
    w["final_norm"] = _gain(seed, _stream_id(-1, "final_norm"), d, gain_std)
    w["layers"] = []
    for l in range(shape.n_layers):
        if layers is not None and l not in layers:
            w["layers"].append(None)
            continue
        lw = {}
        for name, shp in shape.matrix_shapes().items():
            if shape.weight_format == "int4":
                lw[name] = _int4_matrix(seed, _stream_id(l, name), shp, shape.group_size, std)
            else:
                lw[name] = normal_bf16(seed, _stream_id(l, name), shp, std)
        for name in _NORMS:
            lw[name] = _gain(seed, _stream_id(l, name), d, gain_std)
        w["layers"].append(lw)
    return w


def _gain(seed: int, stream: int, d: int, gain_std: float) -> np.ndarray:
    if gain_std <= 0:
        return np.full(d, BF16_ONE, dtype=np.uint16)
    return normal_bf16(seed, stream, (d,), gain_std, mean=1.0)


# --------------------------------------------------------------------------- workloads

def prompts(seed: int, lengths, vocab: int) -> List[np.ndarray]:
    """Token-id prompts, uniform in [0, vocab)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return [rng.integers(0, vocab, size=int(n), dtype=np.int64).astype(np.int32) for n in lengths]


def shared_prefix_prompts(seed: int, lengths, vocab: int, prefix_len: int = 1024) -> List[np.ndarray]:
    """Prompts that share a common prefix: prompt i = prefix[:min(L_i, P)] + own suffix."""
    rng = np.random.Generator(np.random.PCG64(seed))
    prefix = rng.integers(0, vocab, size=prefix_len, dtype=np.int64).astype(np.int32)
    out = []
    for n in lengths:
        n = int(n)
        suf = rng.integers(0, vocab, size=max(0, n - prefix_len), dtype=np.int64).astype(np.int32)
        out.append(np.concatenate([prefix[:min(n, prefix_len)], suf]))
    return out


def uniform_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform on [lo, hi] inclusive."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=n, dtype=np.int64)


def kv_history(shape: ModelShape, seed: int, row: int, n_tokens: int,
               layer: Optional[int] = None, std: Optional[float] = None):
    """Seeded K/V history for one sequence, bf16 bits, layout ``[L, n, Hkv, Dh]``.

    Values are N(0, (weight_std*sqrt(d))^2): the spread a random-init
    projection gives for unit-RMS inputs. With ``layer`` set, only that
    layer's ``[n, Hkv, Dh]`` slice is regenerated (same values)."""
    if std is None:
        std = shape.weight_std * float(np.sqrt(shape.d_model))
    per_layer = n_tokens * shape.kv_dim
    ls = range(shape.n_layers) if layer is None else [layer]
    ks, vs = [], []
    for l in ls:
        ks.append(normal_bf16(seed, 10_000_000 + 2 * row, (n_tokens, shape.n_kv_heads, shape.head_dim),
                              std, offset=l * per_layer))
        vs.append(normal_bf16(seed, 10_000_001 + 2 * row, (n_tokens, shape.n_kv_heads, shape.head_dim),
                              std, offset=l * per_layer))
    if layer is not None:
        return ks[0], vs[0]
    return np.stack(ks), np.stack(vs)
