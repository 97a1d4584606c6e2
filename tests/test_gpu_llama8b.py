"""GPU parity at the full Llama-3-8B shape, in the launch configurations the benchmark times.

One decode step of B = 8 rows whose slabs hold seeded histories with contexts uniform in
[512, 4096] (the benchmark's recipe), with the benchmark's engine limits; every logit of every
row, the greedy ids and the K/V appended at each row's position are compared with the oracle.
"""
import sys

import numpy as np
import pytest

import synth
from gpu_common import assert_logits_close, check_greedy, compare_slab_bits

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_llama8b_shape_decode_step():
    import torch
    import continuous_batching_decode_amd as cbd
    from oracle import OracleModel

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    shape = synth.LLAMA8B
    B = 8
    ctx = synth.uniform_lengths(1, B, 512, 4096).astype(int)
    _say("llama3-8b shape: generating weights; contexts %s" % list(ctx))
    w = synth.make_weights(shape, seed=0)
    gran = cbd.lib().cbd_slab_granule_tokens()
    caps = [int(c) + 16 for c in ctx]
    arena = sum((c + gran - 1) // gran * gran for c in caps) * shape.kv_bytes_per_token()
    eng = cbd.Engine(w, arena_bytes=arena, max_batch=64, max_prefill_tokens=64, max_position=max(caps) + gran)
    orc = OracleModel(w)
    ids, oids = [], []
    for r in range(B):
        k, v = synth.kv_history(shape, 1, r, int(ctx[r]))
        i = eng.alloc(caps[r])
        eng.append(i, torch.from_numpy(k.view(np.int16)).cuda(), torch.from_numpy(v.view(np.int16)).cuda())
        o = orc.new_sequence()
        orc.append_history(o, k, v)
        ids.append(i)
        oids.append(o)
    tok = synth.prompts(2, [B], shape.vocab)[0].astype(np.int64)
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    _say("llama3-8b shape: GPU step")
    eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits, nxt)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    _say("llama3-8b shape: oracle step")
    ref = orc.decode_step_batch(oids, tok)
    errs = assert_logits_close(got, ref, "8b step")
    amb = check_greedy(nxt.cpu().numpy(), ref, errs, "8b step")
    _say("llama3-8b shape: max rel err %.3g, tie-ambiguous rows %d" % (float(np.max(errs / np.max(np.abs(ref), axis=1))), amb))
    assert amb <= 1
    for r in range(B):
        assert eng.length(ids[r]) == int(ctx[r]) + 1
        k, v = eng.read(ids[r], int(ctx[r]), 1)
        torch.cuda.synchronize()
        compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[oids[r]].k)[:, ctx[r]:ctx[r] + 1], "K row %d" % r)
        compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[oids[r]].v)[:, ctx[r]:ctx[r] + 1], "V row %d" % r)
    eng.close()


def test_llama8b_shape_b64_sampled_rows():
    """B = 64 at the full 8B shape, the widest batch the benchmark sweep times, where the products
    take the wide dense tiles. Rows are independent, so the oracle computes 4 sampled rows of the
    batch; their logits, greedy ids and appended K/V are compared. Contexts U[64, 512] keep the
    seeded histories small."""
    import torch
    import continuous_batching_decode_amd as cbd
    from oracle import OracleModel

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    shape = synth.LLAMA8B
    B = 64
    sample = [0, 21, 42, 63]
    ctx = synth.uniform_lengths(31, B, 64, 512).astype(int)
    _say("llama3-8b shape B=64: generating weights")
    w = synth.make_weights(shape, seed=0)
    gran = cbd.lib().cbd_slab_granule_tokens()
    caps = [int(c) + 16 for c in ctx]
    arena = sum((c + gran - 1) // gran * gran for c in caps) * shape.kv_bytes_per_token()
    eng = cbd.Engine(w, arena_bytes=arena, max_batch=64, max_prefill_tokens=64, max_position=max(caps) + gran)
    orc = OracleModel(w)
    ids, oids = [], {}
    for r in range(B):
        k, v = synth.kv_history(shape, 32, r, int(ctx[r]))
        i = eng.alloc(caps[r])
        eng.append(i, torch.from_numpy(k.view(np.int16)).cuda(), torch.from_numpy(v.view(np.int16)).cuda())
        ids.append(i)
        if r in sample:
            o = orc.new_sequence()
            orc.append_history(o, k, v)
            oids[r] = o
    tok = synth.prompts(33, [B], shape.vocab)[0].astype(np.int64)
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    _say("llama3-8b shape B=64: GPU step")
    eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits, nxt)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()[sample]
    _say("llama3-8b shape B=64: oracle step on rows %s" % sample)
    ref = orc.decode_step_batch([oids[r] for r in sample], tok[sample])
    errs = assert_logits_close(got, ref, "8b B=64 sampled rows")
    amb = check_greedy(nxt.cpu().numpy()[sample], ref, errs, "8b B=64 sampled rows")
    assert amb <= 1
    for r in sample:
        assert eng.length(ids[r]) == int(ctx[r]) + 1
        k, v = eng.read(ids[r], int(ctx[r]), 1)
        torch.cuda.synchronize()
        compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[oids[r]].k)[:, ctx[r]:ctx[r] + 1], "K row %d" % r)
        compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[oids[r]].v)[:, ctx[r]:ctx[r] + 1], "V row %d" % r)
    eng.close()
