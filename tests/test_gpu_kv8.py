"""GPU parity of affine 8-bit and 4-bit K/V slabs against the oracle.

Codes and (scale, bias) pairs of given bf16 histories are integer / float32 decisions from identical
inputs, so they must match the oracle's quantization bit for bit. K/V of tokens the model computes come
from the GPU's own projection, whose bf16 value can sit on the other side of a code boundary: the oracle
takes the GPU's stored form as input wherever it is a valid decision for a value within the projection
bound of its own (GpuStoredKV), and fails the test otherwise; every logit follows the rule of the other
parity tests (max |d| <= 1e-2 max |logit| per row), for 8- and 4-bit slabs alike.
"""
import sys

import numpy as np
import pytest

import synth
from gpu_common import MID, GpuStoredKV, assert_logits_close, check_greedy

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a visible GPU"
    return t


@pytest.fixture(scope="module")
def cbd():
    import continuous_batching_decode_amd as m
    m.lib()
    return m


def to_dev_bits(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


FORMATS = ["affine8", "affine4"]


def _engine(cbd, w, shape, tokens, fmt="affine8", **kw):
    per_tok = cbd.kv_bytes_per_token(shape, fmt)
    return cbd.Engine(w, arena_bytes=tokens * per_tok, kv_format=fmt, **kw)


def _quantize(fmt, x):
    from oracle.kvquant import quantize_affine
    return quantize_affine(x, 64, 8 if fmt == "affine8" else 4)


def check_appended(fmt, got_codes, got_sb, want_codes, want_sb, what):
    """K or V the GPU stored ([L, n, Hkv, Dh] codes, [L, n, Hkv, Dh/64, 2] pairs) against the oracle's slab,
    which holds the GPU's form wherever GpuStoredKV accepted it as a valid decision: equal bit for bit."""
    got_sb = np.ascontiguousarray(got_sb, dtype=np.float32)
    want_sb = np.ascontiguousarray(want_sb, dtype=np.float32)
    assert got_codes.shape == want_codes.shape, (what, got_codes.shape, want_codes.shape)
    bad = np.argwhere(got_codes != want_codes)
    assert bad.size == 0, "%s: %d codes differ, first at %s" % (what, len(bad), bad[0].tolist())
    assert np.array_equal(got_sb.view(np.uint32), want_sb.view(np.uint32)), what + ": scale/bias pairs differ"


def _special_history(shape, n, seed):
    """Seeded history with groups that exercise the quantizer's edge cases: constant groups, groups
    on an exact grid, a group with one outlier, and values with exact half-way quotients."""
    k, v = synth.kv_history(shape, seed, 0, n)
    rng = np.random.default_rng(seed)
    f = lambda x: synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    for arr in (k, v):
        if n > 0:
            arr[:, 0, :, :] = f(np.full(arr[:, 0].shape, 0.375))                  # constant groups
        if n > 1:
            codes = rng.integers(0, 256, arr[:, 1].shape)
            arr[:, 1] = f(-1.0 + codes * 2.0 ** -7)                               # on a grid
        if n > 2:
            x = rng.normal(0, 0.01, arr[:, 2].shape)
            x[..., 5] = 40.0
            arr[:, 2] = f(x)                                                      # one outlier per head
        if n > 3:
            # lo = 0, hi = 255 * 2^-6: quotients (x - lo) / s land on halves for x = (c + 0.5) 2^-6
            x = (rng.integers(0, 255, arr[:, 3].shape) + 0.5) * 2.0 ** -6
            x[..., 0::64] = 0.0
            x[..., 1::64] = 255 * 2.0 ** -6
            arr[:, 3] = f(x)
    return k, v


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [synth.TINY, MID], ids=["dh64-g2", "dh128-g4"])
def test_kv8_append_matches_oracle_quantization(torch, cbd, shape, fmt):
    _say("kv append codes", shape.name, fmt)
    w = synth.make_weights(shape, seed=1)
    eng = _engine(cbd, w, shape, 8 * 256, fmt, max_position=4096)
    a, b = eng.alloc(700), eng.alloc(300)
    k, v = _special_history(shape, 650, 21)
    # appends of ragged sizes that end inside a 32-key block and across a 256-token granule
    for lo, hi in ((0, 5), (5, 37), (37, 400), (400, 650)):
        eng.append(a, to_dev_bits(torch, k[:, lo:hi]), to_dev_bits(torch, v[:, lo:hi]))
    kb, vb = synth.kv_history(shape, 22, 1, 300)
    eng.append(b, to_dev_bits(torch, kb), to_dev_bits(torch, vb))
    for sid, kk, vv, start, n in ((a, k, v, 0, 650), (b, kb, vb, 17, 100)):
        codes, sb = eng.kvslab_read_q8(sid, start, n)
        torch.cuda.synchronize()
        codes, sb = codes.cpu().numpy(), sb.cpu().numpy()
        for which, x in ((0, kk), (1, vv)):
            rc, rsb = _quantize(fmt, x[:, start:start + n])
            assert np.array_equal(codes[:, :, which], rc), "codes %d" % which
            assert np.array_equal(sb[:, :, which].view(np.uint32), rsb.view(np.uint32)), "pairs %d" % which
    with pytest.raises(cbd.CbdError) as ei:
        eng.read(a, 0, 1)
    assert ei.value.status == cbd.CBD_E_UNSUPPORTED
    eng.close()


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [MID, synth.TINY], ids=["dh128-g4", "dh64-g2"])
def test_kv8_ragged_decode_matches_oracle(torch, cbd, shape, fmt):
    """Ragged histories (one-item and split rows), three teacher-forced decode steps."""
    from oracle import OracleModel, dequantize_affine8, greedy
    _say("kv ragged decode", shape.name, fmt)
    w = synth.make_weights(shape, seed=3, gain_std=0.1)
    ctx = [0, 1, 31, 32, 33, 700, 2999, 4095]
    eng = _engine(cbd, w, shape, 64 * 256, fmt, max_batch=16, max_prefill_tokens=64, max_position=8192)
    orc = OracleModel(w, cache_all_layers=True, kv_format=fmt)
    ids, oids = [], []
    for r, n in enumerate(ctx):
        i = eng.alloc(n + 4)
        o = orc.new_sequence()
        if n:
            k, v = _special_history(shape, n, 30 + r)
            eng.append(i, to_dev_bits(torch, k), to_dev_bits(torch, v))
            orc.append_history(o, k, v)
        ids.append(i)
        oids.append(o)
    before = [eng.kvslab_read_q8(i, 0, n) if n else None for i, n in zip(ids, ctx)]
    tok = synth.prompts(12, [len(ctx)], shape.vocab)[0].astype(np.int64)
    logits = torch.empty((len(ctx), shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(len(ctx), dtype=torch.int32, device="cuda")
    stored = GpuStoredKV(fmt)
    orc.stored_override = stored
    for step in range(3):
        eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits, nxt)
        stored.capture(torch, eng, [(i, o, n + step, 1) for i, o, n in zip(ids, oids, ctx)])
        ref = orc.decode_step_batch(oids, tok)
        torch.cuda.synchronize()
        errs = assert_logits_close(logits.cpu().numpy(), ref, "step %d" % step)
        check_greedy(nxt.cpu().numpy(), ref, errs, "step %d" % step)
        tok = greedy(ref)
    stored.assert_consumed()
    _say("  stored forms checked %d, taken from the GPU %d" % (stored.checked, stored.replaced))
    for r, (i, o, n) in enumerate(zip(ids, oids, ctx)):
        codes, sb = eng.kvslab_read_q8(i, 0, n + 3)
        torch.cuda.synchronize()
        codes, sb = codes.cpu().numpy(), sb.cpu().numpy()
        if n:  # the history is untouched by the steps
            assert np.array_equal(codes[:, :n], before[r][0].cpu().numpy())
            assert np.array_equal(sb[:, :n], before[r][1].cpu().numpy())
        # the three appended tokens
        s = orc.seqs[o]
        for which, oc, osb in ((0, s.k, s.k_sb), (1, s.v, s.v_sb)):
            check_appended(fmt, codes[:, n:, which], sb[:, n:, which], np.stack(oc)[:, n:], np.stack(osb)[:, n:],
                           "row %d kv %d" % (r, which))
            assert np.all(codes[:, n:, which].reshape(-1, 64).min(axis=1) == 0)  # min of each group -> 0
    eng.close()


@pytest.mark.parametrize("fmt", FORMATS)
def test_kv8_long_context_sampled_rows(torch, cbd, fmt):
    """Llama-3-8B attention shape (32 query / 8 KV heads, Dh 128) at long contexts, one layer, three
    rows of different lengths (many splits per row); a decode step against the oracle."""
    from oracle import OracleModel
    _say("kv long context", fmt)
    shape = synth.ModelShape("kv8-long", 1, 4096, 32, 8, 128, 512, 1024, 500000.0)
    w = synth.make_weights(shape, seed=5, gain_std=0.1)
    ctx = [32767, 9000, 511]
    eng = _engine(cbd, w, shape, sum((c + 256) // 256 * 256 for c in ctx), fmt, max_batch=8, max_position=32768)
    orc = OracleModel(w, cache_all_layers=True, kv_format=fmt)
    ids, oids = [], []
    for r, n in enumerate(ctx):
        i = eng.alloc(n + 1)
        o = orc.new_sequence()
        k, v = synth.kv_history(shape, 40, r, n)
        eng.append(i, to_dev_bits(torch, k), to_dev_bits(torch, v))
        orc.append_history(o, k, v)
        ids.append(i)
        oids.append(o)
    tok = np.array([3, 500, 77], dtype=np.int64)
    logits = torch.empty((len(ctx), shape.vocab), dtype=torch.float32, device="cuda")
    eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits)
    stored = GpuStoredKV(fmt)
    stored.capture(torch, eng, [(i, o, n, 1) for i, o, n in zip(ids, oids, ctx)])
    orc.stored_override = stored
    ref = orc.decode_step_batch(oids, tok)
    stored.assert_consumed()
    torch.cuda.synchronize()
    assert_logits_close(logits.cpu().numpy(), ref, "kv8 long")
    eng.close()


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [MID, synth.TINY], ids=["dh128-g4", "dh64-g2"])
def test_kv8_prefill_continuation_and_decode(torch, cbd, shape, fmt):
    """Segmented prefill into affine 8-bit slabs (mixed lengths, one segment continuing its sequence in a
    second call after decode steps), every call's logits and the stored K/V against the oracle."""
    from oracle import OracleModel, dequantize_affine8, greedy
    _say("kv prefill", shape.name, fmt)
    w = synth.make_weights(shape, seed=7, gain_std=0.1)
    lens = [1, 31, 32, 33, 100, 115]
    prompts = synth.prompts(23, lens + [45], shape.vocab)
    eng = _engine(cbd, w, shape, 16 * 256, fmt, max_batch=8, max_prefill_tokens=512, max_position=1024)
    orc = OracleModel(w, cache_all_layers=True, kv_format=fmt)
    ids = [eng.alloc(256) for _ in lens]
    oids = [orc.new_sequence() for _ in lens]
    stored = GpuStoredKV(fmt)
    orc.stored_override = stored

    def prefill(rows, segs, what):
        toks = torch.from_numpy(np.concatenate(segs).astype(np.int32)).cuda()
        lg = torch.empty((len(rows), shape.vocab), dtype=torch.float32, device="cuda")
        nx = torch.empty(len(rows), dtype=torch.int32, device="cuda")
        t0 = [eng.length(ids[r]) for r in rows]
        eng.prefill_segmented([ids[r] for r in rows], [len(x) for x in segs], toks, lg, nx)
        stored.capture(torch, eng, [(ids[r], oids[r], t, len(x)) for r, t, x in zip(rows, t0, segs)])
        ref = orc.prefill_segmented([oids[r] for r in rows], segs)
        torch.cuda.synchronize()
        errs = assert_logits_close(lg.cpu().numpy(), ref, what)
        check_greedy(nx.cpu().numpy(), ref, errs, what)
        return greedy(ref)

    rows = list(range(len(lens)))
    tok = prefill(rows, prompts[:len(lens)], "prefill")
    lg = torch.empty((len(rows), shape.vocab), dtype=torch.float32, device="cuda")
    for step in range(2):
        t0 = [eng.length(ids[r]) for r in rows]
        eng.decode_step_batch([ids[r] for r in rows], torch.from_numpy(tok.astype(np.int32)).cuda(), lg)
        stored.capture(torch, eng, [(ids[r], oids[r], t, 1) for r, t in zip(rows, t0)])
        ref = orc.decode_step_batch([oids[r] for r in rows], tok)
        torch.cuda.synchronize()
        assert_logits_close(lg.cpu().numpy(), ref, "decode %d" % step)
        tok = greedy(ref)
    prefill([4], [prompts[-1]], "continuation")  # 100 + 2 decoded + 45 more prompt tokens
    stored.assert_consumed()
    _say("  stored forms checked %d, taken from the GPU %d" % (stored.checked, stored.replaced))
    for r in rows:
        n = orc.seqs[oids[r]].length
        assert eng.length(ids[r]) == n
        codes, sb = eng.kvslab_read_q8(ids[r], 0, n)
        torch.cuda.synchronize()
        codes, sb = codes.cpu().numpy(), sb.cpu().numpy()
        s = orc.seqs[oids[r]]
        for which, oc, osb in ((0, s.k, s.k_sb), (1, s.v, s.v_sb)):
            check_appended(fmt, codes[:, :, which], sb[:, :, which], np.stack(oc), np.stack(osb),
                           "row %d kv %d" % (r, which))
    eng.close()
