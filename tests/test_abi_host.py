"""Host-side tests of the C ABI: exports, slab bookkeeping and argument validation.

A host-only context (no device memory, no kernels) runs the same validation
and bookkeeping code as a device context, so every error path here is forced
from the host; none of them launches anything.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def cbd():
    import continuous_batching_decode_amd as m
    if not os.path.exists(m.LIB_PATH):
        from continuous_batching_decode_amd import build
        build.build()
    m.lib()
    return m


def header_functions():
    text = open(os.path.join(ROOT, "include", "cbd.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_header_symbol(cbd):
    names = header_functions()
    assert len(names) >= 15
    assert sorted(cbd.EXPORTS) == names
    lib = cbd.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_kv_bytes_and_granule(cbd):
    cfg = cbd.model_config(synth.LLAMA8B, 40000)
    assert cbd.lib().cbd_kv_bytes_per_token(ctypes.byref(cfg)) == 131072
    assert cbd.lib().cbd_slab_granule_tokens() == 256


def make(cbd, shape=synth.TINY, granules=8, **kw):
    g = cbd.lib().cbd_slab_granule_tokens()
    return cbd.Engine({"shape": shape}, arena_bytes=granules * g * shape.kv_bytes_per_token(), host_only=True,
                      max_position=kw.pop("max_position", 4096), **kw)


def test_alloc_free_len_and_reuse(cbd):
    e = make(cbd)
    a = e.alloc(100)
    b = e.alloc(300)
    assert (a, b) == (0, 1)
    assert e.length(a) == 0 and e.capacity(a) == 256 and e.capacity(b) == 512
    st = e.stats()
    assert st["live_seqs"] == 2 and st["arena_bytes_used"] == 3 * 256 * synth.TINY.kv_bytes_per_token()
    e.free(a)
    assert e.alloc(1) == 0  # ids are reused
    with pytest.raises(cbd.CbdError) as ei:
        e.length(7)
    assert ei.value.status == cbd.CBD_E_BADSEQ
    e.free(b)
    with pytest.raises(cbd.CbdError) as ei:
        e.free(b)
    assert ei.value.status == cbd.CBD_E_BADSEQ


def test_arena_exhaustion_and_coalescing(cbd):
    e = make(cbd, granules=4)
    ids = [e.alloc(256) for _ in range(4)]
    with pytest.raises(cbd.CbdError) as ei:
        e.alloc(1)
    assert ei.value.status == cbd.CBD_E_NOSPACE  # caller queues and retries later
    e.free(ids[1])
    e.free(ids[2])
    # the two freed neighbours coalesce into one run of 2 granules
    big = e.alloc(512)
    assert e.capacity(big) == 512
    with pytest.raises(cbd.CbdError) as ei:
        e.alloc(5 * 256)
    assert ei.value.status == cbd.CBD_E_CAPACITY  # larger than the whole arena: can never fit
    for i in (ids[0], ids[3], big):
        e.free(i)
    assert e.stats()["arena_bytes_used"] == 0
    assert e.capacity(e.alloc(4 * 256)) == 1024


def test_capacity_above_rope_table(cbd):
    e = make(cbd, granules=64, max_position=1000)
    with pytest.raises(cbd.CbdError) as ei:
        e.alloc(1001)
    assert ei.value.status == cbd.CBD_E_CAPACITY
    assert e.capacity(e.alloc(1000)) == 1000  # rounded capacity is clipped to the table


def test_decode_validation_without_state_change(cbd):
    e = make(cbd, max_batch=4)
    a, b = e.alloc(10), e.alloc(10)
    P = 4096  # stands in for device pointers; a host-only context never dereferences them
    assert e.decode_step_batch_raw([], P, P) == cbd.CBD_OK  # B = 0 is a no-op
    assert e.decode_step_batch_raw([a, a], P, P) == cbd.CBD_E_INVAL  # duplicate id
    assert e.decode_step_batch_raw([a, 9], P, P) == cbd.CBD_E_BADSEQ
    assert e.decode_step_batch_raw([a, b, 0, 1, 0], P, P) == cbd.CBD_E_INVAL  # B > max_batch
    assert e.decode_step_batch_raw([a], None, P) == cbd.CBD_E_INVAL
    assert e.decode_step_batch_raw([a, b], P, P) == cbd.CBD_E_NODEVICE  # valid, but no device here
    assert e.length(a) == 0 and e.length(b) == 0
    e.free(b)
    assert e.decode_step_batch_raw([a, b], P, P) == cbd.CBD_E_BADSEQ


def test_prefill_validation(cbd):
    e = make(cbd, max_prefill_tokens=100, max_segments=3)
    a, b = e.alloc(50), e.alloc(300)
    P = 4096
    assert e.prefill_segmented_raw([], [], P, P) == cbd.CBD_OK
    assert e.prefill_segmented_raw([a, b], [3, 0], P, P) == cbd.CBD_E_INVAL  # zero-length segment
    assert e.prefill_segmented_raw([a, a], [3, 4], P, P) == cbd.CBD_E_INVAL  # duplicate
    assert e.prefill_segmented_raw([a, b], [60, 41], P, P) == cbd.CBD_E_INVAL  # total above the limit
    assert e.prefill_segmented_raw([a], [257], P, P) == cbd.CBD_E_CAPACITY  # longer than the slab
    assert e.prefill_segmented_raw([a, b, 0, 1], [1, 1, 1, 1], P, P) == cbd.CBD_E_INVAL  # K > max_segments
    assert e.prefill_segmented_raw([a, 5], [1, 1], P, P) == cbd.CBD_E_BADSEQ
    assert e.prefill_segmented_raw([a, b], [10, 20], P, P) == cbd.CBD_E_NODEVICE
    assert e.length(a) == 0 and e.length(b) == 0


def test_sample_validation(cbd):
    """sample_top_p checks rows and every row's parameters before anything is enqueued."""
    import ctypes
    e = make(cbd)
    P = 4096  # stands in for 16-byte aligned device pointers
    F, U = ctypes.c_float, ctypes.c_uint64

    def call(rows, temps, tops, logits=P, out=P):
        n = max(1, len(temps))
        return e.lib.sample_top_p(e.ctx, logits, rows, (F * n)(*temps), (F * n)(*tops), (U * n)(*([1] * n)),
                                  (U * n)(*([0] * n)), out, None)
    assert call(0, [], []) == cbd.CBD_OK
    assert call(65, [1.0] * 65, [0.9] * 65) == cbd.CBD_E_INVAL  # more than 64 rows
    assert call(2, [1.0, -0.5], [0.9, 0.9]) == cbd.CBD_E_INVAL  # negative temperature
    assert call(1, [float("inf")], [0.9]) == cbd.CBD_E_INVAL
    assert call(1, [float("nan")], [0.9]) == cbd.CBD_E_INVAL
    assert call(2, [1.0, 1.0], [0.9, 0.0]) == cbd.CBD_E_INVAL  # top_p outside (0, 1]
    assert call(1, [1.0], [1.5]) == cbd.CBD_E_INVAL
    assert call(1, [1.0], [0.9], logits=P + 4) == cbd.CBD_E_INVAL  # unaligned logits
    assert call(1, [1.0], [0.9], out=None) == cbd.CBD_E_INVAL
    assert call(2, [0.0, 0.7], [1.0, 0.5]) == cbd.CBD_E_NODEVICE  # valid, but no device here


def test_create_rejects_bad_shapes(cbd):
    from dataclasses import replace
    for bad in (replace(synth.TINY, head_dim=96), replace(synth.TINY, n_heads=3),
                replace(synth.TINY, d_model=200), replace(synth.TINY, vocab=1000),
                replace(synth.TINY, n_heads=16, n_kv_heads=2)):
        with pytest.raises(cbd.CbdError) as ei:
            make(cbd, shape=bad)
        assert ei.value.status == cbd.CBD_E_INVAL
    with pytest.raises(cbd.CbdError):
        make(cbd, max_batch=65)
    with pytest.raises(cbd.CbdError):
        make(cbd, max_segments=0)


def unpack_int4_reference(packed, aux, n, k):
    """Decode the packed layout as the header documents it (independent of the packer's loops)."""
    codes = np.zeros((n, k), dtype=np.uint8)
    words = packed.reshape(n // 16, k // 128, 64, 4)  # [row tile, block, lane, word]
    for lane in range(64):
        r, g = lane % 16, lane // 16
        for j in range(4):
            w = words[:, :, lane, j].astype(np.uint64)  # [row tile, block]
            for e in range(8):
                nib = (e // 2) + 4 * (e % 2)
                vals = ((w >> np.uint64(4 * nib)) & np.uint64(15)).astype(np.uint8)
                rows = np.arange(n // 16) * 16 + r
                cols = np.arange(k // 128) * 128 + 32 * j + 8 * g + e
                codes[np.ix_(rows, cols)] = vals
    scale = aux[:, :, 0].T.copy()
    bias = aux[:, :, 1].T.copy()
    return codes, scale, bias


def test_int4_packing_layout(cbd):
    m = synth._int4_matrix(3, 5, (32, 256), 64, 0.02)
    packed, aux = cbd.pack_int4(m["codes"], m["scale"], m["bias"])
    assert packed.shape == (32 * 256 // 8,) and aux.shape == (4, 32, 2)
    codes, scale, bias = unpack_int4_reference(packed, aux, 32, 256)
    assert np.array_equal(codes, m["codes"])
    assert np.array_equal(scale, m["scale"]) and np.array_equal(bias, m["bias"])
    with pytest.raises(cbd.CbdError):
        cbd.pack_int4(np.full((16, 256), 16, np.uint8), m["scale"][:16], m["bias"][:16])


def test_affine8_kv_format_host(cbd):
    """Affine 8-bit slabs: bytes per token, arena accounting and the calls that reject the format."""
    assert cbd.kv_bytes_per_token(synth.LLAMA8B, "affine8") == 32 * 2 * 8 * (128 + 2 * 8)
    assert cbd.kv_bytes_per_token(synth.TINY, "affine8") == 2 * 2 * 2 * (64 + 8)
    assert cbd.kv_bytes_per_token(synth.LLAMA8B, "bf16") == synth.LLAMA8B.kv_bytes_per_token()
    assert cbd.kv_bytes_per_token(synth.LLAMA8B, "affine4") == 32 * 2 * 8 * (64 + 2 * 8)
    g = cbd.lib().cbd_slab_granule_tokens()
    per_tok = cbd.kv_bytes_per_token(synth.TINY, "affine8")
    e = cbd.Engine({"shape": synth.TINY}, arena_bytes=4 * g * per_tok, host_only=True, max_position=4096,
                   kv_format="affine8")
    a = e.alloc(2 * g)
    assert e.stats()["arena_bytes_used"] == 2 * g * per_tok
    b = e.alloc(2 * g)
    with pytest.raises(cbd.CbdError) as ei:
        e.alloc(1)
    assert ei.value.status == cbd.CBD_E_NOSPACE
    lib = cbd.lib()
    ids = (ctypes.c_int32 * 1)(a)
    lens = (ctypes.c_int32 * 1)(4)
    assert lib.prefill_segmented(e.ctx, ids, lens, 1, 256, 256, None, None) == cbd.CBD_E_NODEVICE
    assert lib.kvslab_read(e.ctx, a, 0, 0, 256, 256, None) == cbd.CBD_E_UNSUPPORTED
    assert lib.kvslab_read_q8(e.ctx, a, 0, 0, 256, 256, None) == cbd.CBD_OK
    assert lib.kvslab_read_q8(e.ctx, a, 0, 1, 256, 256, None) == cbd.CBD_E_CAPACITY
    assert lib.kvslab_read_q8(e.ctx, b + 5, 0, 0, 256, 256, None) == cbd.CBD_E_BADSEQ
    e.free(a)
    e.free(b)
    bf = make(cbd)
    s = bf.alloc(10)
    assert lib.kvslab_read_q8(bf.ctx, s, 0, 0, 256, 256, None) == cbd.CBD_E_UNSUPPORTED
    cfg = cbd.model_config(synth.TINY, 4096)
    cfg.kv_format = 5
    lim = cbd.Limits(8, 64, 8, 1)
    ctx = ctypes.c_void_p()
    assert lib.cbd_create(ctypes.byref(cfg), None, ctypes.byref(lim), None, 1 << 20, ctypes.byref(ctx)) == cbd.CBD_E_INVAL


def test_fork_bookkeeping_host(cbd):
    """kvslab_fork: validation, the fork's own granules, and a freed parent kept until its forks go."""
    e = make(cbd, granules=8)
    per_gran = 256 * synth.TINY.kv_bytes_per_token()
    par = e.alloc(300)  # 2 granules
    kid = e.fork(par, 0, 600)  # prefix 0: 3 granules of its own
    assert e.length(kid) == 0 and e.capacity(kid) == 768
    assert e.stats()["arena_bytes_used"] == 5 * per_gran
    for args, status in (((par, 1, 100), cbd.CBD_E_INVAL),      # prefix beyond the parent's length
                         ((par, 0, 0), cbd.CBD_E_INVAL),        # no room after the prefix
                         ((kid, 0, 100), cbd.CBD_E_INVAL),      # fork of a fork
                         ((par, 0, 5000), cbd.CBD_E_CAPACITY),  # beyond max_position
                         ((par, 0, 4 * 256), cbd.CBD_E_NOSPACE),
                         ((77, 0, 10), cbd.CBD_E_BADSEQ)):
        with pytest.raises(cbd.CbdError) as ei:
            e.fork(*args)
        assert ei.value.status == status, args
    e.free(par)  # the fork still reads it: id retired, memory kept
    with pytest.raises(cbd.CbdError) as ei:
        e.length(par)
    assert ei.value.status == cbd.CBD_E_BADSEQ
    st = e.stats()
    assert st["live_seqs"] == 1 and st["arena_bytes_used"] == 5 * per_gran
    other = e.alloc(10)
    assert other not in (par, kid)  # the retired id is not reused while its memory is held
    e.free(kid)  # the last fork: the parent's granules return too
    assert e.stats()["arena_bytes_used"] == 1 * per_gran
    e.free(other)
    assert e.stats()["arena_bytes_used"] == 0
    assert e.alloc(8 * 256) == 0  # the whole arena is one free run again
