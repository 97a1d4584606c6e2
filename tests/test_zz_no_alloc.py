"""The scratch-free greedy selection (cbd_greedy_argmax_noalloc) against the context's greedy_argmax.

Both run the same selection rule (lowest id among each row's maxima); the scratch-free entry point keeps
its kernel's partials and arrival counters in the library's static device array instead of a context
workspace. Calls in a row share that array: a second, smaller call (fewer rows, a shorter vocabulary)
and a third, larger one again must each give exactly the context entry point's tokens.
"""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _logits(seed, rows, vocab):
    x = synth.normal_f32(seed, 1, (rows, vocab), 3.0)
    rng = np.random.default_rng(seed)
    for r in range(0, rows, 3):  # ties of the row maximum at several ids
        ids = rng.choice(vocab, size=4, replace=False)
        x[r, ids] = x[r].max() + 1.0
    x[1 % rows] = 0.5  # every id tied
    if rows > 2:
        x[2, : vocab // 2] = np.nan  # NaNs weigh nothing
    return x


def _engine(cbd, vocab):
    shape = synth.ModelShape("argmax-v%d" % vocab, 1, 256, 4, 2, 64, 512, vocab, 10000.0)
    return cbd.Engine(synth.make_weights(shape, seed=1), arena_bytes=1 << 20, max_batch=64, max_prefill_tokens=64,
                      max_position=256)


def test_greedy_argmax_noalloc_matches_context_entry_point():
    import torch
    import continuous_batching_decode_amd as cbd
    from oracle import greedy

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    engines = {v: _engine(cbd, v) for v in (128256, 1024)}
    for call, (rows, vocab) in enumerate(((64, 128256), (5, 1024), (33, 128256))):
        _say("noalloc argmax call %d: rows %d, vocab %d" % (call, rows, vocab))
        x = _logits(40 + call, rows, vocab)
        xd = torch.from_numpy(x).cuda()
        got = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
        want = torch.full((rows,), -2, dtype=torch.int32, device="cuda")
        cbd.greedy_argmax_noalloc(xd, got)
        engines[vocab].greedy_argmax(xd, want)
        torch.cuda.synchronize()
        g, w = got.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(g, w), (call, g, w)
        assert np.array_equal(g, greedy(np.where(np.isnan(x), -np.inf, x))), call
    # sizes beyond the scratch are refused before any launch
    big = torch.zeros((65, 1024), dtype=torch.float32, device="cuda")
    with pytest.raises(cbd.CbdError) as e:
        cbd.greedy_argmax_noalloc(big, torch.empty(65, dtype=torch.int32, device="cuda"))
    assert e.value.status == cbd.CBD_E_INVAL
    for eng in engines.values():
        eng.close()
