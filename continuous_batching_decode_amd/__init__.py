"""Python binding of libcbd.so (ctypes), the C-ABI library declared in include/cbd.h.

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI. PyTorch provides device memory and streams.
There is no fallback: importing this package on a machine without the built
library raises, and every entry point raises on a non-OK status.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcbd.so")

CBD_OK, CBD_E_INVAL, CBD_E_NOSPACE, CBD_E_CAPACITY, CBD_E_BADSEQ, CBD_E_HIP, CBD_E_NODEVICE = 0, -1, -2, -3, -4, -5, -6
CBD_E_UNSUPPORTED = -7
STATUS_NAMES = {0: "CBD_OK", -1: "CBD_E_INVAL", -2: "CBD_E_NOSPACE", -3: "CBD_E_CAPACITY", -4: "CBD_E_BADSEQ",
                -5: "CBD_E_HIP", -6: "CBD_E_NODEVICE", -7: "CBD_E_UNSUPPORTED"}
WEIGHTS_BF16, WEIGHTS_INT4 = 0, 1
KV_BF16, KV_AFFINE8, KV_AFFINE4 = 0, 1, 2
KV_FORMATS = {"bf16": KV_BF16, "affine8": KV_AFFINE8, "affine4": KV_AFFINE4}

# every symbol include/cbd.h declares
EXPORTS = ["cbd_kv_bytes_per_token", "cbd_slab_granule_tokens", "cbd_create", "cbd_destroy", "cbd_last_error",
           "cbd_stats", "kvslab_alloc", "kvslab_free", "kvslab_len", "kvslab_capacity", "kvslab_append",
           "kvslab_read", "decode_step_batch", "prefill_segmented", "greedy_argmax", "cbd_linear", "cbd_pack_int4",
           "cbd_profile_begin", "cbd_profile_end", "cbd_pack_bf16", "sample_top_p", "kvslab_read_q8", "kvslab_fork",
           "cbd_greedy_argmax_noalloc"]

KERNEL_KINDS = ["embed", "norm", "qkv", "rope_append", "attention", "attn_combine", "o_proj", "gate_up", "down",
                "lm_head", "argmax", "sample"]


class CbdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status


class ModelConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn_dim", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("weight_format", ctypes.c_int32), ("max_position", ctypes.c_int32),
                ("kv_format", ctypes.c_int32)]


class Matrix(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("aux", ctypes.c_void_p)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("wq", Matrix), ("wk", Matrix), ("wv", Matrix), ("wo", Matrix),
                ("ffn_norm", ctypes.c_void_p), ("w_gate", Matrix), ("w_up", Matrix), ("w_down", Matrix)]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", Matrix),
                ("layers", ctypes.POINTER(LayerWeights))]


class Limits(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("max_prefill_tokens", ctypes.c_int32),
                ("max_segments", ctypes.c_int32), ("host_only", ctypes.c_int32)]


class KernelTime(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("total_ms", ctypes.c_double), ("bytes", ctypes.c_double),
                ("flops", ctypes.c_double)]


class Stats(ctypes.Structure):
    _fields_ = [("live_seqs", ctypes.c_int64), ("arena_bytes", ctypes.c_int64), ("arena_bytes_used", ctypes.c_int64),
                ("decode_steps", ctypes.c_int64), ("decode_rows", ctypes.c_int64), ("prefill_calls", ctypes.c_int64),
                ("prefill_tokens", ctypes.c_int64)]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError("libcbd.so is not built (%s); run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    P, i32, i64, vp, sz = ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    ctx_p = vp
    sig = {
        "cbd_kv_bytes_per_token": (sz, [P(ModelConfig)]),
        "cbd_slab_granule_tokens": (i32, []),
        "cbd_create": (i32, [P(ModelConfig), P(Weights), P(Limits), vp, sz, P(ctx_p)]),
        "cbd_destroy": (i32, [ctx_p]),
        "cbd_last_error": (ctypes.c_char_p, []),
        "cbd_stats": (i32, [ctx_p, P(Stats)]),
        "kvslab_alloc": (i32, [ctx_p, i32, P(i32)]),
        "kvslab_free": (i32, [ctx_p, i32]),
        "kvslab_len": (i32, [ctx_p, i32, P(i32)]),
        "kvslab_capacity": (i32, [ctx_p, i32, P(i32)]),
        "kvslab_append": (i32, [ctx_p, i32, i32, vp, vp, vp]),
        "kvslab_read": (i32, [ctx_p, i32, i32, i32, vp, vp, vp]),
        "kvslab_read_q8": (i32, [ctx_p, i32, i32, i32, vp, vp, vp]),
        "kvslab_fork": (i32, [ctx_p, i32, i32, i32, P(i32), vp]),
        "decode_step_batch": (i32, [ctx_p, P(i32), i32, vp, vp, vp, vp]),
        "prefill_segmented": (i32, [ctx_p, P(i32), P(i32), i32, vp, vp, vp, vp]),
        "greedy_argmax": (i32, [ctx_p, vp, i32, vp, vp]),
        "cbd_greedy_argmax_noalloc": (i32, [vp, i32, i32, vp, vp]),
        "sample_top_p": (i32, [ctx_p, vp, i32, P(ctypes.c_float), P(ctypes.c_float), P(ctypes.c_uint64),
                               P(ctypes.c_uint64), vp, vp]),
        "cbd_linear": (i32, [ctx_p, P(Matrix), i32, i32, vp, i32, vp, i32, vp]),
        "cbd_pack_int4": (i32, [vp, vp, vp, i64, i64, vp, vp]),
        "cbd_profile_begin": (i32, [ctx_p, ctypes.c_uint32, i32, i32]),
        "cbd_pack_bf16": (i32, [vp, i64, i64, vp, vp]),
        "cbd_profile_end": (i32, [ctx_p, P(KernelTime)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


def _check(status: int) -> None:
    if status != CBD_OK:
        raise CbdError(status, lib().cbd_last_error().decode())


def _ids(seq: Sequence[int]):
    arr = (ctypes.c_int32 * len(seq))(*[int(s) for s in seq])
    return arr


def kv_bytes_per_token(shape, kv_format: str = "bf16") -> int:
    """Slab bytes per token over all layers, as the library counts them."""
    cfg = model_config(shape, 1, kv_format)
    return int(lib().cbd_kv_bytes_per_token(ctypes.byref(cfg)))


def model_config(shape, max_position: int, kv_format: str = "bf16") -> ModelConfig:
    """C config from a shape object (attributes as in synth.ModelShape); kv_format "bf16", "affine8" or
    "affine4"."""
    return ModelConfig(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                       shape.ffn_dim, shape.vocab, float(shape.rms_eps), float(shape.rope_theta),
                       WEIGHTS_INT4 if shape.weight_format == "int4" else WEIGHTS_BF16, int(max_position),
                       KV_FORMATS[kv_format])


def pack_int4(codes: np.ndarray, scale: np.ndarray, bias: np.ndarray):
    """Host packing into the library's int4 layout (see cbd_pack_int4)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    bias = np.ascontiguousarray(bias, dtype=np.uint16)
    n, k = codes.shape
    packed = np.empty((n * k // 8,), dtype=np.uint32)
    aux = np.empty((k // 64, n, 2), dtype=np.uint16)
    _check(lib().cbd_pack_int4(codes.ctypes.data, scale.ctypes.data, bias.ctypes.data, n, k,
                               packed.ctypes.data, aux.ctypes.data))
    return packed, aux


def pack_bf16_device(w_rowmajor_dev, stream=None):
    """Device-side repack of a row-major bf16 matrix (int16 tensor [N, K]) into the streaming layout."""
    import torch
    out = torch.empty_like(w_rowmajor_dev)
    n, k = w_rowmajor_dev.shape
    _check(lib().cbd_pack_bf16(w_rowmajor_dev.data_ptr(), int(n), int(k), out.data_ptr(), _stream_ptr(stream)))
    return out


def _tensor(t, dtype: str, min_numel: int, name: str) -> int:
    """Device pointer of a tensor passed to the library, after checking what the C ABI assumes of it:
    a contiguous tensor on the GPU of the expected element type holding at least min_numel elements.
    Raises ValueError otherwise (the library would read or write out of bounds)."""
    import torch
    want = getattr(torch, dtype)
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != want:
        raise ValueError("%s must be %s, not %s" % (name, dtype, str(t.dtype).replace("torch.", "")))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() < min_numel:
        raise ValueError("%s holds %d elements, %d needed" % (name, t.numel(), min_numel))
    return t.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def greedy_argmax_noalloc(logits_dev, tokens_dev, stream=None) -> None:
    """Context-free greedy selection over rows of logits (float32 [rows, vocab] device tensor) into
    tokens_dev (int32 [rows]); the library allocates nothing (cbd_greedy_argmax_noalloc)."""
    if logits_dev.dim() != 2:
        raise ValueError("logits must be [rows, vocab]")
    rows, vocab = int(logits_dev.shape[0]), int(logits_dev.shape[1])
    lp = _tensor(logits_dev, "float32", rows * vocab, "logits")
    tp = _tensor(tokens_dev, "int32", rows, "tokens")
    _check(lib().cbd_greedy_argmax_noalloc(lp, rows, vocab, tp, _stream_ptr(stream)))


class Engine:
    """One context: device weights, a KV arena and the C-ABI entry points.

    ``weights`` is a dict as produced by ``synth.make_weights`` (bf16 bit
    patterns as uint16, int4 matrices as {codes, scale, bias}). Weights are
    copied to the device once (model loading); the per-step work runs only
    in the library."""

    def __init__(self, weights: Dict, arena_bytes: int, max_batch: int = 64, max_prefill_tokens: int = 1024,
                 max_segments: int = 64, max_position: Optional[int] = None, host_only: bool = False,
                 device: str = "cuda", kv_format: str = "bf16"):
        self.shape = shape = weights["shape"]
        self.lib = lib()
        if max_position is None:
            max_position = 8192
        self.kv_format = kv_format
        self.cfg = model_config(shape, max_position, kv_format)
        self.limits = Limits(max_batch, max_prefill_tokens, max_segments, 1 if host_only else 0)
        self._keep: List = []
        self.arena = None
        arena_ptr = None
        wts = None
        if not host_only:
            import torch
            self.device = torch.device(device)
            self.arena = torch.empty(int(arena_bytes), dtype=torch.uint8, device=self.device)
            arena_ptr = self.arena.data_ptr()
            wts = self._upload_weights(weights)
        ctx = ctypes.c_void_p()
        _check(self.lib.cbd_create(ctypes.byref(self.cfg), ctypes.byref(wts) if wts is not None else None,
                                   ctypes.byref(self.limits), arena_ptr, int(arena_bytes), ctypes.byref(ctx)))
        self.ctx = ctx

    # -- model loading (host -> device copies only)
    def _dev(self, a: np.ndarray):
        import torch
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        elif a.dtype == np.uint32:
            a = a.view(np.int32)
        t = torch.from_numpy(a).to(self.device)
        self._keep.append(t)
        return t.data_ptr()

    def _mat(self, m) -> Matrix:
        if isinstance(m, dict):
            packed, aux = pack_int4(m["codes"], m["scale"], m["bias"])
            return Matrix(self._dev(packed), self._dev(aux))
        import torch
        rowmajor = torch.from_numpy(np.ascontiguousarray(m).view(np.int16)).to(self.device)
        packed = pack_bf16_device(rowmajor)
        torch.cuda.synchronize()
        del rowmajor
        self._keep.append(packed)
        return Matrix(packed.data_ptr(), None)

    def _upload_weights(self, w: Dict) -> Weights:
        layers = (LayerWeights * self.shape.n_layers)()
        for l, lw in enumerate(w["layers"]):
            layers[l] = LayerWeights(self._dev(lw["attn_norm"]), self._mat(lw["wq"]), self._mat(lw["wk"]),
                                     self._mat(lw["wv"]), self._mat(lw["wo"]), self._dev(lw["ffn_norm"]),
                                     self._mat(lw["w_gate"]), self._mat(lw["w_up"]), self._mat(lw["w_down"]))
        self._layers = layers
        return Weights(self._dev(w["embed"]), self._dev(w["final_norm"]), self._mat(w["lm_head"]), layers)

    def close(self) -> None:
        if getattr(self, "ctx", None):
            _check(self.lib.cbd_destroy(self.ctx))
            self.ctx = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass

    # -- slabs
    def alloc(self, capacity_tokens: int) -> int:
        out = ctypes.c_int32()
        _check(self.lib.kvslab_alloc(self.ctx, int(capacity_tokens), ctypes.byref(out)))
        return out.value

    def free(self, seq_id: int) -> None:
        _check(self.lib.kvslab_free(self.ctx, int(seq_id)))

    def length(self, seq_id: int) -> int:
        out = ctypes.c_int32()
        _check(self.lib.kvslab_len(self.ctx, int(seq_id), ctypes.byref(out)))
        return out.value

    def capacity(self, seq_id: int) -> int:
        out = ctypes.c_int32()
        _check(self.lib.kvslab_capacity(self.ctx, int(seq_id), ctypes.byref(out)))
        return out.value

    def fork(self, parent: int, prefix_len: int, capacity_tokens: int, stream=None) -> int:
        """A new sequence that shares the parent's first prefix_len positions."""
        out = ctypes.c_int32()
        st = None if self.arena is None else _stream_ptr(stream)  # a host-only context copies nothing
        _check(self.lib.kvslab_fork(self.ctx, int(parent), int(prefix_len), int(capacity_tokens), ctypes.byref(out),
                                    st))
        return out.value

    def append(self, seq_id: int, k_dev, v_dev, stream=None) -> None:
        """k_dev, v_dev: device int16 tensors holding bf16 bits, [L, n, Hkv, Dh]."""
        s = self.shape
        n = int(k_dev.shape[1]) if k_dev.dim() == 4 else -1
        if tuple(k_dev.shape) != (s.n_layers, n, s.n_kv_heads, s.head_dim) or tuple(v_dev.shape) != tuple(k_dev.shape):
            raise ValueError("k and v must both be [L, n, Hkv, Dh] = [%d, n, %d, %d]" % (s.n_layers, s.n_kv_heads,
                                                                                      s.head_dim))
        kp = _tensor(k_dev, "int16", k_dev.numel(), "k")
        vp = _tensor(v_dev, "int16", v_dev.numel(), "v")
        _check(self.lib.kvslab_append(self.ctx, int(seq_id), n, kp, vp, _stream_ptr(stream)))

    def read(self, seq_id: int, start: int, n: int, stream=None):
        """Slab positions [start, start+n) as device int16 tensors (bf16 bits) [L, n, Hkv, Dh]."""
        import torch
        s = self.shape
        k = torch.empty((s.n_layers, n, s.n_kv_heads, s.head_dim), dtype=torch.int16, device=self.device)
        v = torch.empty_like(k)
        _check(self.lib.kvslab_read(self.ctx, int(seq_id), int(start), int(n), k.data_ptr(), v.data_ptr(),
                                    _stream_ptr(stream)))
        return k, v

    def kvslab_read_q8(self, seq_id: int, start: int, n: int, stream=None):
        """Stored form of an affine slab: codes uint8 [L, n, 2, Hkv, Dh] (one per byte) and (scale, bias)
        float32 [L, n, 2, Hkv, Dh/64, 2] (device tensors)."""
        import torch
        s = self.shape
        codes = torch.empty((s.n_layers, n, 2, s.n_kv_heads, s.head_dim), dtype=torch.uint8, device=self.device)
        sb = torch.empty((s.n_layers, n, 2, s.n_kv_heads, s.head_dim // 64, 2), dtype=torch.float32,
                         device=self.device)
        _check(self.lib.kvslab_read_q8(self.ctx, int(seq_id), int(start), int(n), codes.data_ptr(), sb.data_ptr(),
                                       _stream_ptr(stream)))
        return codes, sb

    def stats(self) -> Dict[str, int]:
        st = Stats()
        _check(self.lib.cbd_stats(self.ctx, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in Stats._fields_}

    # -- hot path
    def decode_step_batch(self, seq_ids: Sequence[int], last_tokens_dev, logits_dev, next_tokens_dev=None,
                          stream=None) -> None:
        """last_tokens_dev: int32 [B]; logits_dev: float32 [B, vocab]; next_tokens_dev: int32 [B] or None."""
        B, V = len(seq_ids), self.shape.vocab
        tp = _tensor(last_tokens_dev, "int32", B, "last_tokens")
        lp = _tensor(logits_dev, "float32", B * V, "logits")
        np_ = _tensor(next_tokens_dev, "int32", B, "next_tokens") if next_tokens_dev is not None else None
        _check(self.lib.decode_step_batch(self.ctx, _ids(seq_ids), B, tp, lp, np_, _stream_ptr(stream)))

    def prefill_segmented(self, seq_ids: Sequence[int], seg_lens: Sequence[int], tokens_dev, last_logits_dev,
                          next_tokens_dev=None, stream=None) -> None:
        """tokens_dev: int32 [sum(seg_lens)]; last_logits_dev: float32 [K, vocab]; next_tokens_dev: int32 [K]."""
        K, V = len(seq_ids), self.shape.vocab
        tp = _tensor(tokens_dev, "int32", sum(int(n) for n in seg_lens), "tokens")
        lp = _tensor(last_logits_dev, "float32", K * V, "last_logits")
        np_ = _tensor(next_tokens_dev, "int32", K, "next_tokens") if next_tokens_dev is not None else None
        _check(self.lib.prefill_segmented(self.ctx, _ids(seq_ids), _ids(seg_lens), K, tp, lp, np_,
                                          _stream_ptr(stream)))

    def greedy_argmax(self, logits_dev, tokens_dev, stream=None) -> None:
        """logits_dev: float32 [rows, vocab]; tokens_dev: int32 [rows]."""
        rows = int(logits_dev.shape[0])
        lp = _tensor(logits_dev, "float32", rows * self.shape.vocab, "logits")
        tp = _tensor(tokens_dev, "int32", rows, "tokens")
        _check(self.lib.greedy_argmax(self.ctx, lp, rows, tp, _stream_ptr(stream)))

    def sample_top_p(self, logits_dev, temperature, top_p, seeds, sample_index, tokens_dev, stream=None) -> None:
        """Seeded temperature / top-p sampling of each logits row (host lists of per-row parameters)."""
        rows = int(logits_dev.shape[0])
        for name, xs in (("temperature", temperature), ("top_p", top_p), ("seeds", seeds),
                         ("sample_index", sample_index)):
            if len(xs) < rows:
                raise ValueError("%s: %d values for %d rows" % (name, len(xs), rows))
        lp = _tensor(logits_dev, "float32", rows * self.shape.vocab, "logits")
        tp = _tensor(tokens_dev, "int32", rows, "tokens")
        F = ctypes.c_float * max(rows, 1)
        U = ctypes.c_uint64 * max(rows, 1)
        _check(self.lib.sample_top_p(self.ctx, lp, rows, F(*[float(x) for x in temperature[:rows]]),
                                     F(*[float(x) for x in top_p[:rows]]), U(*[int(x) for x in seeds[:rows]]),
                                     U(*[int(x) for x in sample_index[:rows]]), tp, _stream_ptr(stream)))

    def linear(self, w_ptrs: Matrix, N: int, K: int, x_dev, y_dev, splits: int = 0, stream=None) -> None:
        """y_dev[b] = W x_dev[b]; x_dev fp32 [rows, K] device tensor, y_dev fp32 [rows, N]."""
        rows = int(x_dev.shape[0])
        if x_dev.dim() != 2 or int(x_dev.shape[1]) != int(K):
            raise ValueError("x must be [rows, K] with K = %d" % K)
        xp = _tensor(x_dev, "float32", rows * int(K), "x")
        yp = _tensor(y_dev, "float32", rows * int(N), "y")
        _check(self.lib.cbd_linear(self.ctx, ctypes.byref(w_ptrs), int(N), int(K), xp, rows, yp, int(splits),
                                   _stream_ptr(stream)))

    # -- per-kernel event timing
    def profile_begin(self, kinds: Sequence[str], max_launches: int = 1 << 16, every: int = 1) -> None:
        mask = 0
        for k in kinds:
            mask |= 1 << KERNEL_KINDS.index(k)
        _check(self.lib.cbd_profile_begin(self.ctx, mask, int(max_launches), int(every)))

    def profile_end(self) -> Dict[str, Dict[str, float]]:
        out = (KernelTime * len(KERNEL_KINDS))()
        _check(self.lib.cbd_profile_end(self.ctx, out))
        return {k: {"launches": out[i].launches, "total_ms": out[i].total_ms, "bytes": out[i].bytes,
                    "flops": out[i].flops} for i, k in enumerate(KERNEL_KINDS) if out[i].launches}

    # -- host-only calls without torch (validation tests)
    def decode_step_batch_raw(self, seq_ids: Sequence[int], tokens_ptr=None, logits_ptr=None) -> int:
        return self.lib.decode_step_batch(self.ctx, _ids(seq_ids), len(seq_ids), tokens_ptr, logits_ptr, None, None)

    def prefill_segmented_raw(self, seq_ids: Sequence[int], seg_lens: Sequence[int], tokens_ptr=None,
                              logits_ptr=None) -> int:
        return self.lib.prefill_segmented(self.ctx, _ids(seq_ids), _ids(seg_lens), len(seq_ids), tokens_ptr,
                                          logits_ptr, None, None)
