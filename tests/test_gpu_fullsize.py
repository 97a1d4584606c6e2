"""GPU parity at the full sizes of the long-context, segmented-prefill and 4-bit-weight workloads.

- bf16 decode over 32768-token histories at the Llama-3-8B attention shape (32 query / 8 KV heads,
  Dh 128): the step's planner then cuts rows into work items of over a thousand keys, RoPE runs at
  positions near 32k, and a second case reaches the 64-split cap of one row.
- prefill_segmented at d_model 4096 (Llama-3-8B layer widths) over 16 prompts with lengths uniform in
  [64, 1024] (about 7.8k tokens): MFMA dense products over many 64-row blocks, block-diagonal causal
  attention over segments up to 1024 tokens; every segment's last logits and the stored K/V.
- a decode step of the Mistral-7B-shaped model with 4-bit affine weights at full widths (vocab 32768)
  over histories of 1024..8192 tokens.
One or two layers each keep the oracle's float64 run within a minute; every layer runs the same
kernels in the same launch configurations as the full-depth model.
"""
import sys
import time
from dataclasses import replace

import numpy as np
import pytest

import synth
from gpu_common import assert_logits_close, check_greedy, compare_slab_bits

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


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


# one layer of the Llama-3-8B attention shape (the FFN and vocabulary are small: they do not change the
# attention kernel's work items)
ATTN8B = synth.ModelShape("llama3-8b-attention-1l", 1, 4096, 32, 8, 128, 512, 1024, 500000.0)


@pytest.mark.parametrize("ctx", [[32768] * 8, [16383, 1000, 5]], ids=["8x32768", "split-cap"])
def test_bf16_decode_long_context(torch, cbd, ctx):
    """Two teacher-forced decode steps over seeded bf16 histories: every logit, the greedy ids and the
    K/V appended at positions ctx and ctx + 1."""
    from oracle import OracleModel, greedy
    _say("bf16 long-context decode, contexts %s" % ctx)
    shape = ATTN8B
    w = synth.make_weights(shape, seed=15, gain_std=0.1)
    gran = cbd.lib().cbd_slab_granule_tokens()
    caps = [c + 2 for c in ctx]
    arena = sum((c + gran - 1) // gran * gran for c in caps) * shape.kv_bytes_per_token()
    eng = cbd.Engine(w, arena_bytes=arena, max_batch=8, max_prefill_tokens=64, max_position=max(caps) + gran)
    orc = OracleModel(w, cache_all_layers=True)
    ids, oids = [], []
    for r, n in enumerate(ctx):
        k, v = synth.kv_history(shape, 70, r, n)
        i = eng.alloc(caps[r])
        eng.append(i, to_dev_bits(torch, k), to_dev_bits(torch, v))
        o = orc.new_sequence()
        orc.append_history(o, k, v)
        ids.append(i)
        oids.append(o)
        del k, v
    tok = synth.prompts(71, [len(ctx)], shape.vocab)[0].astype(np.int64)
    logits = torch.empty((len(ctx), shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(len(ctx), dtype=torch.int32, device="cuda")
    for step in range(2):
        eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits, nxt)
        torch.cuda.synchronize()
        t0 = time.time()
        ref = orc.decode_step_batch(oids, tok)
        errs = assert_logits_close(logits.cpu().numpy(), ref, "step %d" % step)
        check_greedy(nxt.cpu().numpy(), ref, errs, "step %d" % step)
        _say("  step %d: max rel err %.3g (oracle %.1f s)" % (
            step, float(np.max(errs / np.max(np.abs(ref), axis=1))), time.time() - t0))
        tok = greedy(ref)
    for r, n in enumerate(ctx):
        assert eng.length(ids[r]) == n + 2
        k, v = eng.read(ids[r], n, 2)
        torch.cuda.synchronize()
        compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[oids[r]].k)[:, n:n + 2], "K row %d" % r)
        compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[oids[r]].v)[:, n:n + 2], "V row %d" % r)
    eng.close()


def test_prefill_segmented_llama8b_width(torch, cbd):
    """16 prompts, lengths uniform in [64, 1024], into fresh slabs in one call: every segment's last
    logits and greedy id, and the stored K/V of three segments."""
    from oracle import OracleModel
    shape = replace(synth.LLAMA8B, name="llama3-8b-width-2l", n_layers=2, vocab=32768)
    lens = [int(x) for x in synth.uniform_lengths(5, 16, 64, 1024)]
    _say("prefill at d_model 4096: %d segments, %d tokens" % (len(lens), sum(lens)))
    w = synth.make_weights(shape, seed=16)
    prompts = synth.prompts(17, lens, shape.vocab)
    gran = cbd.lib().cbd_slab_granule_tokens()
    arena = sum((n + gran - 1) // gran * gran for n in lens) * shape.kv_bytes_per_token()
    eng = cbd.Engine(w, arena_bytes=arena, max_batch=16, max_prefill_tokens=8192, max_segments=16,
                     max_position=1024 + gran)
    orc = OracleModel(w, cache_all_layers=True)
    ids = [eng.alloc(n) for n in lens]
    oids = [orc.new_sequence() for _ in lens]
    toks = torch.from_numpy(np.concatenate(prompts).astype(np.int32)).cuda()
    logits = torch.empty((len(lens), shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(len(lens), dtype=torch.int32, device="cuda")
    eng.prefill_segmented(ids, lens, toks, logits, nxt)
    torch.cuda.synchronize()
    t0 = time.time()
    ref = orc.prefill_segmented(oids, prompts)
    errs = assert_logits_close(logits.cpu().numpy(), ref, "prefill")
    amb = check_greedy(nxt.cpu().numpy(), ref, errs, "prefill")
    _say("  max rel err %.3g, tie-ambiguous rows %d (oracle %.1f s)" % (
        float(np.max(errs / np.max(np.abs(ref), axis=1))), amb, time.time() - t0))
    for j in (int(np.argmin(lens)), int(np.argmax(lens)), 5):
        assert eng.length(ids[j]) == lens[j]
        k, v = eng.read(ids[j], 0, lens[j])
        torch.cuda.synchronize()
        compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[oids[j]].k), "K segment %d" % j)
        compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[oids[j]].v), "V segment %d" % j)
    eng.close()


def test_int4_decode_mistral7b_width(torch, cbd):
    """Two teacher-forced decode steps of the 4-bit model at Mistral-7B widths (vocab 32768), B = 8 rows
    over seeded histories of 1024..8192 tokens: every logit, greedy ids, appended K/V."""
    from oracle import OracleModel, greedy
    shape = replace(synth.MISTRAL7B_INT4, name="mistral7b-width-int4-2l", n_layers=2)
    ctx = [int(x) for x in synth.uniform_lengths(4, 8, 1024, 8192)]
    _say("int4 decode at Mistral-7B widths, contexts %s" % ctx)
    w = synth.make_weights(shape, seed=3)
    gran = cbd.lib().cbd_slab_granule_tokens()
    caps = [c + 2 for c in ctx]
    arena = sum((c + gran - 1) // gran * gran for c in caps) * shape.kv_bytes_per_token()
    eng = cbd.Engine(w, arena_bytes=arena, max_batch=16, max_prefill_tokens=64, max_position=8192 + gran)
    orc = OracleModel(w, cache_all_layers=True)
    ids, oids = [], []
    for r, n in enumerate(ctx):
        k, v = synth.kv_history(shape, 4, r, n)
        i = eng.alloc(caps[r])
        eng.append(i, to_dev_bits(torch, k), to_dev_bits(torch, v))
        o = orc.new_sequence()
        orc.append_history(o, k, v)
        ids.append(i)
        oids.append(o)
    tok = synth.prompts(72, [len(ctx)], shape.vocab)[0].astype(np.int64)
    logits = torch.empty((len(ctx), shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(len(ctx), dtype=torch.int32, device="cuda")
    for step in range(2):
        eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits, nxt)
        torch.cuda.synchronize()
        t0 = time.time()
        ref = orc.decode_step_batch(oids, tok)
        errs = assert_logits_close(logits.cpu().numpy(), ref, "step %d" % step)
        check_greedy(nxt.cpu().numpy(), ref, errs, "step %d" % step)
        _say("  step %d: max rel err %.3g (oracle %.1f s)" % (
            step, float(np.max(errs / np.max(np.abs(ref), axis=1))), time.time() - t0))
        tok = greedy(ref)
    for r, n in enumerate(ctx):
        k, v = eng.read(ids[r], n, 2)
        torch.cuda.synchronize()
        compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[oids[r]].k)[:, n:n + 2], "K row %d" % r)
        compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[oids[r]].v)[:, n:n + 2], "V row %d" % r)
    eng.close()
