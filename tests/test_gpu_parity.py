"""GPU parity: the HIP path through the C ABI against the CPU oracle.

All inputs come from ``synth`` (seeded); expected values come only from the
oracle (or from an fp64 matmul of the same bf16 / int4 values for the
standalone weight-streaming product).
"""
import sys

import numpy as np
import pytest

import synth
from gpu_common import MID, MID_INT4, WIDE, assert_logits_close, check_greedy, compare_slab_bits

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


# ----------------------------------------------------------------------------- weight-streaming product

LINEAR_HOST = synth.ModelShape("linear-host", 1, 512, 4, 1, 128, 14336, 256, 10000.0)


@pytest.fixture(scope="module")
def linear_engines(torch, cbd):
    from dataclasses import replace
    engs = {}
    for fmt in ("bf16", "int4"):
        sh = replace(LINEAR_HOST, weight_format=fmt)
        engs[fmt] = cbd.Engine(synth.make_weights(sh, seed=98), arena_bytes=1 << 20, max_batch=64,
                               max_prefill_tokens=64, max_position=256)
    yield engs
    for e in engs.values():
        e.close()


# Activations enter as fp32 and are carried as bf16 hi + lo planes (about 16
# significant bits); weights are exact bf16 and products accumulate in fp32,
# so the result is within a few 1e-6 of the float64 product of the same values.
LINEAR_RTOL = 2e-5


@pytest.mark.parametrize("N,K", [(6144, 4096), (4096, 14336), (1024, 256), (512, 1024)])
@pytest.mark.parametrize("rows", [1, 7, 16, 24, 33, 64])
def test_linear_bf16(torch, cbd, linear_engines, N, K, rows):
    _say("linear bf16 N=%d K=%d rows=%d" % (N, K, rows))
    eng = linear_engines["bf16"]
    W = synth.normal_bf16(7, N + K, (N, K), 0.02)
    X = synth.normal_f32(8, rows, (rows, K), 1.0)
    wd, xd = cbd.pack_bf16_device(to_dev_bits(torch, W)), torch.from_numpy(X).cuda()
    y = torch.empty((rows, N), dtype=torch.float32, device="cuda")
    eng.linear(cbd.Matrix(wd.data_ptr(), None), N, K, xd, y)
    torch.cuda.synchronize()
    ref = X.astype(np.float64) @ synth.bf16_bits_to_f32(W).astype(np.float64).T
    got = y.cpu().numpy()
    err = np.max(np.abs(got - ref))
    assert err <= LINEAR_RTOL * np.max(np.abs(ref)), err


@pytest.mark.parametrize("rows", [40, 64])
def test_linear_bf16_wide_n(torch, cbd, linear_engines, rows):
    """A product with enough weight rows (98304) for 256-row dense tiles without a K split."""
    N, K = 98304, 256
    _say("linear bf16 N=%d K=%d rows=%d" % (N, K, rows))
    eng = linear_engines["bf16"]
    W = synth.normal_bf16(17, N + K, (N, K), 0.02)
    X = synth.normal_f32(18, rows, (rows, K), 1.0)
    wd, xd = cbd.pack_bf16_device(to_dev_bits(torch, W)), torch.from_numpy(X).cuda()
    y = torch.empty((rows, N), dtype=torch.float32, device="cuda")
    eng.linear(cbd.Matrix(wd.data_ptr(), None), N, K, xd, y)
    torch.cuda.synchronize()
    ref = X.astype(np.float64) @ synth.bf16_bits_to_f32(W).astype(np.float64).T
    err = np.max(np.abs(y.cpu().numpy() - ref))
    assert err <= LINEAR_RTOL * np.max(np.abs(ref)), err


@pytest.mark.parametrize("waves,rows", [(4, 1), (8, 8), (16, 8), (4, 33), (8, 64)])
def test_linear_bf16_forced_k_split(torch, cbd, linear_engines, waves, rows):
    """The k-split kernel with 4, 8 or 16 waves per tile forced through cbd_linear."""
    N, K = 4096, 4096
    _say("linear bf16 forced k split waves=%d rows=%d" % (waves, rows))
    eng = linear_engines["bf16"]
    W = synth.normal_bf16(27, N + K, (N, K), 0.02)
    X = synth.normal_f32(28, rows, (rows, K), 1.0)
    wd, xd = cbd.pack_bf16_device(to_dev_bits(torch, W)), torch.from_numpy(X).cuda()
    y = torch.empty((rows, N), dtype=torch.float32, device="cuda")
    eng.linear(cbd.Matrix(wd.data_ptr(), None), N, K, xd, y, splits=-waves)
    torch.cuda.synchronize()
    ref = X.astype(np.float64) @ synth.bf16_bits_to_f32(W).astype(np.float64).T
    err = np.max(np.abs(y.cpu().numpy() - ref))
    assert err <= LINEAR_RTOL * np.max(np.abs(ref)), err
    # 16 waves take one row group only: 9 rows are rejected before any launch
    with pytest.raises(cbd.CbdError) as e:
        eng.linear(cbd.Matrix(wd.data_ptr(), None), N, K, torch.from_numpy(np.tile(X[:1], (9, 1))).cuda(),
                   torch.empty((9, N), dtype=torch.float32, device="cuda"), splits=-16)
    assert e.value.status == cbd.CBD_E_INVAL


@pytest.mark.parametrize("splits", [1, 2, 7, 16])
@pytest.mark.parametrize("N,K,rows", [(4096, 14336, 8), (4096, 14336, 1), (1024, 14336, 33)])
def test_linear_bf16_splits(torch, cbd, linear_engines, N, K, rows, splits):
    """Every split of K over workgroups gives the product (fixed-order reduction of partial tiles)."""
    _say("linear bf16 splits=%d N=%d K=%d rows=%d" % (splits, N, K, rows))
    eng = linear_engines["bf16"]
    W = synth.normal_bf16(17, N + K, (N, K), 0.02)
    X = synth.normal_f32(18, rows, (rows, K), 1.0)
    wd, xd = cbd.pack_bf16_device(to_dev_bits(torch, W)), torch.from_numpy(X).cuda()
    y = torch.empty((rows, N), dtype=torch.float32, device="cuda")
    eng.linear(cbd.Matrix(wd.data_ptr(), None), N, K, xd, y, splits=splits)
    torch.cuda.synchronize()
    y2 = torch.empty_like(y)
    eng.linear(cbd.Matrix(wd.data_ptr(), None), N, K, xd, y2, splits=splits)  # counters were reset
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    torch.cuda.synchronize()
    ref = X.astype(np.float64) @ synth.bf16_bits_to_f32(W).astype(np.float64).T
    err = np.max(np.abs(y.cpu().numpy() - ref))
    assert err <= LINEAR_RTOL * np.max(np.abs(ref)), err


@pytest.mark.parametrize("N,K", [(6144, 4096), (4096, 14336), (512, 512)])
@pytest.mark.parametrize("rows", [1, 5, 16, 40, 64])
def test_linear_int4(torch, cbd, linear_engines, N, K, rows):
    _say("linear int4 N=%d K=%d rows=%d" % (N, K, rows))
    eng = linear_engines["int4"]
    m = synth._int4_matrix(9, N + K, (N, K), 64, 0.02)
    packed, aux = cbd.pack_int4(m["codes"], m["scale"], m["bias"])
    pd = torch.from_numpy(packed.view(np.int32)).cuda()
    ad = to_dev_bits(torch, aux)
    X = synth.normal_f32(10, rows, (rows, K), 1.0)
    xd = torch.from_numpy(X).cuda()
    y = torch.empty((rows, N), dtype=torch.float32, device="cuda")
    eng.linear(cbd.Matrix(pd.data_ptr(), ad.data_ptr()), N, K, xd, y)
    torch.cuda.synchronize()
    from oracle import dequant_int4
    Wd = dequant_int4(m["codes"], m["scale"], m["bias"], 64)
    ref = X.astype(np.float64) @ Wd.T
    err = np.max(np.abs(y.cpu().numpy() - ref))
    assert err <= LINEAR_RTOL * np.max(np.abs(ref)), err


# ----------------------------------------------------------------------------- slabs and argmax

def test_pack_bf16_layout(torch, cbd):
    """The device packer writes exactly the documented streaming layout (checked on the host)."""
    N, K = 48, 96
    W = (np.arange(N * K, dtype=np.uint32) % 60000).astype(np.uint16).reshape(N, K)
    got = cbd.pack_bf16_device(to_dev_bits(torch, W)).cpu().numpy().view(np.uint16).reshape(-1)
    ref = np.empty(N * K, dtype=np.uint16)
    for t in range(N // 16):
        for f in range(K // 32):
            for l in range(64):
                off = ((t * (K // 32) + f) * 64 + l) * 8
                ref[off:off + 8] = W[16 * t + l % 16, 32 * f + 8 * (l // 16): 32 * f + 8 * (l // 16) + 8]
    assert np.array_equal(got, ref)


def test_slab_append_read_roundtrip(torch, cbd):
    _say("slab append/read roundtrip")
    w = synth.make_weights(synth.TINY, seed=0)
    eng = cbd.Engine(w, arena_bytes=16 * 256 * synth.TINY.kv_bytes_per_token(), max_position=4096)
    a = eng.alloc(700)
    b = eng.alloc(300)
    k, v = synth.kv_history(synth.TINY, 5, 0, 650)
    eng.append(a, to_dev_bits(torch, k[:, :400]), to_dev_bits(torch, v[:, :400]))
    eng.append(a, to_dev_bits(torch, k[:, 400:]), to_dev_bits(torch, v[:, 400:]))
    kb, vb = synth.kv_history(synth.TINY, 5, 1, 300)
    eng.append(b, to_dev_bits(torch, kb), to_dev_bits(torch, vb))
    assert eng.length(a) == 650 and eng.length(b) == 300
    rk, rv = eng.read(a, 0, 650)
    torch.cuda.synchronize()
    assert np.array_equal(rk.cpu().numpy().view(np.uint16), k)
    assert np.array_equal(rv.cpu().numpy().view(np.uint16), v)
    rk, rv = eng.read(b, 17, 100)
    assert np.array_equal(rk.cpu().numpy().view(np.uint16), kb[:, 17:117])
    with pytest.raises(cbd.CbdError):
        eng.append(b, to_dev_bits(torch, kb[:, :257]), to_dev_bits(torch, vb[:, :257]))  # 300 + 257 > 512
    assert eng.length(b) == 300
    eng.close()


def test_greedy_argmax_ties(torch, cbd):
    _say("argmax ties")
    from oracle import greedy
    w = synth.make_weights(synth.TINY, seed=0)
    eng = cbd.Engine(w, arena_bytes=1 << 20, max_position=256)
    V = synth.TINY.vocab
    rng = np.random.default_rng(0)
    L = rng.integers(-5, 5, size=(9, V)).astype(np.float32)  # many exact ties
    L[3, :] = 2.0
    L[4, 1000:] = 7.0
    L[5, 17] = 100.0
    L[5, 900] = 100.0
    ld = torch.from_numpy(L).cuda()
    out = torch.empty(9, dtype=torch.int32, device="cuda")
    eng.greedy_argmax(ld, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), greedy(L.astype(np.float64)))
    eng.close()


# ----------------------------------------------------------------------------- whole step vs oracle

def _prefill_both(torch, cbd, eng, orc, lengths, prompts, cap):
    ids = [eng.alloc(cap) for _ in lengths]
    oids = [orc.new_sequence() for _ in lengths]
    toks = torch.from_numpy(np.concatenate(prompts).astype(np.int32)).cuda()
    logits = torch.empty((len(lengths), eng.shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(len(lengths), dtype=torch.int32, device="cuda")
    eng.prefill_segmented(ids, lengths, toks, logits, nxt)
    ref = orc.prefill_segmented(oids, prompts)
    torch.cuda.synchronize()
    return ids, oids, logits.cpu().numpy(), nxt.cpu().numpy(), ref


@pytest.mark.parametrize("gain_std", [0.0, 0.1])
def test_tiny_prefill_and_decode_teacher_forced(torch, cbd, gain_std):
    """The small decoder: segmented prefill {17,5,33,1} then 8 greedy decode steps at B=4."""
    _say("tiny teacher-forced gain_std=%g" % gain_std)
    from oracle import OracleModel, greedy
    shape = synth.TINY
    w = synth.make_weights(shape, seed=0, gain_std=gain_std)
    lengths = [17, 5, 33, 1]
    prompts = synth.prompts(100, lengths, shape.vocab)
    eng = cbd.Engine(w, arena_bytes=32 * 256 * shape.kv_bytes_per_token(), max_batch=8, max_prefill_tokens=256,
                     max_position=1024)
    orc = OracleModel(w, cache_all_layers=True)
    ids, oids, got, gtok, ref = _prefill_both(torch, cbd, eng, orc, lengths, prompts, 64)
    errs = assert_logits_close(got, ref, "prefill")
    check_greedy(gtok, ref, errs, "prefill")
    tok = greedy(ref)
    logits = torch.empty((4, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(4, dtype=torch.int32, device="cuda")
    for step in range(8):
        eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits, nxt)
        ref = orc.decode_step_batch(oids, tok)
        torch.cuda.synchronize()
        errs = assert_logits_close(logits.cpu().numpy(), ref, "step %d" % step)
        check_greedy(nxt.cpu().numpy(), ref, errs, "step %d" % step)
        tok = greedy(ref)
    for i, o, n in zip(ids, oids, lengths):
        assert eng.length(i) == n + 8 == orc.seqs[o].length
        k, v = eng.read(i, 0, n + 8)
        torch.cuda.synchronize()
        compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[o].k), "K slab %d" % i)
        compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[o].v), "V slab %d" % i)
    eng.close()


def test_tiny_free_running_trajectory(torch, cbd):
    """Free-running greedy: the GPU feeds its own argmax back on the device for 8 steps. The oracle
    follows the GPU's trajectory (each step it consumes the tokens the GPU consumed), so every step's
    logits are compared; each GPU token must be the oracle's greedy choice, except at a step whose
    oracle top-1/top-2 margin lies within the tie band of that row's error (a tie-ambiguous step, where
    either token is correct). The trajectory then goes on from the GPU's token on both sides."""
    _say("tiny free-running")
    from oracle import OracleModel, greedy
    shape = synth.TINY
    w = synth.make_weights(shape, seed=0)
    lengths = [17, 5, 33, 1]
    prompts = synth.prompts(100, lengths, shape.vocab)
    eng = cbd.Engine(w, arena_bytes=32 * 256 * shape.kv_bytes_per_token(), max_batch=8, max_prefill_tokens=256,
                     max_position=1024)
    orc = OracleModel(w, cache_all_layers=True)
    ids, oids, got, gtok, ref = _prefill_both(torch, cbd, eng, orc, lengths, prompts, 64)
    errs = assert_logits_close(got, ref, "prefill")
    ambiguous = check_greedy(gtok, ref, errs, "prefill")
    differ = int(np.sum(gtok != greedy(ref)))
    tok_dev = torch.from_numpy(gtok.astype(np.int32)).cuda()
    logits = torch.empty((4, shape.vocab), dtype=torch.float32, device="cuda")
    for step in range(8):
        fed = tok_dev.cpu().numpy().astype(np.int64)  # what the GPU consumes this step (its own argmax)
        nxt = torch.empty(4, dtype=torch.int32, device="cuda")
        eng.decode_step_batch(ids, tok_dev, logits, nxt)
        tok_dev = nxt
        ref = orc.decode_step_batch(oids, fed)
        torch.cuda.synchronize()
        errs = assert_logits_close(logits.cpu().numpy(), ref, "step %d" % step)
        g = nxt.cpu().numpy()
        ambiguous += check_greedy(g, ref, errs, "step %d" % step)  # fails on a non-ambiguous difference
        differ += int(np.sum(g != greedy(ref)))
    _say("free-running: %d tie-ambiguous row-steps, %d tokens differing from the oracle's choice" % (ambiguous, differ))
    assert differ <= ambiguous
    eng.close()


def test_ragged_long_history_decode(torch, cbd):
    """Seeded ragged histories (split attention path), GQA G=4, Dh=128; 2 teacher-forced steps."""
    _say("ragged long-history decode")
    from oracle import OracleModel, greedy
    shape = MID
    w = synth.make_weights(shape, seed=3, gain_std=0.1)
    ctx = [0, 1, 63, 64, 65, 700, 2999, 4095]
    eng = cbd.Engine(w, arena_bytes=64 * 256 * shape.kv_bytes_per_token(), max_batch=16, max_prefill_tokens=64,
                     max_position=8192)
    orc = OracleModel(w, cache_all_layers=True)
    ids, oids = [], []
    for r, n in enumerate(ctx):
        i = eng.alloc(n + 4)
        o = orc.new_sequence()
        if n:
            k, v = synth.kv_history(shape, 11, r, n)
            eng.append(i, to_dev_bits(torch, k), to_dev_bits(torch, v))
            orc.append_history(o, k, v)
        ids.append(i)
        oids.append(o)
    tok = synth.prompts(12, [len(ctx)], shape.vocab)[0].astype(np.int64)
    logits = torch.empty((len(ctx), shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(len(ctx), dtype=torch.int32, device="cuda")
    for step in range(2):
        eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits, nxt)
        ref = orc.decode_step_batch(oids, tok)
        torch.cuda.synchronize()
        errs = assert_logits_close(logits.cpu().numpy(), ref, "step %d" % step)
        check_greedy(nxt.cpu().numpy(), ref, errs, "step %d" % step)
        tok = greedy(ref)
    for i, o, n in zip(ids, oids, ctx):
        k, v = eng.read(i, n, 2)
        torch.cuda.synchronize()
        compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[o].k)[:, n:n + 2], "K")
        compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[o].v)[:, n:n + 2], "V")
    # a row's result does not depend on the other rows of the batch
    solo = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    eng2 = cbd.Engine(w, arena_bytes=64 * 256 * shape.kv_bytes_per_token(), max_batch=16, max_position=8192)
    i = eng2.alloc(ctx[5] + 4)
    k, v = eng.read(ids[5], 0, ctx[5] + 2)
    eng2.append(i, k, v)
    eng2.decode_step_batch([i], torch.from_numpy(tok[5:6].astype(np.int32)).cuda(), solo)
    eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits, nxt)
    torch.cuda.synchronize()
    assert_logits_close(solo.cpu().numpy(), logits.cpu().numpy()[5:6], "batched vs solo")
    eng.close()
    eng2.close()


@pytest.mark.parametrize("B,shape", [(24, WIDE), (32, MID), (40, MID), (64, MID), (64, WIDE)],
                         ids=["wide-24", "mid-32", "mid-40", "mid-64", "wide-64"])
def test_wide_batch_decode(torch, cbd, B, shape):
    """Decode steps of 17..64 rows (dense projection tiles of 32 or 64 rows; K split over workgroups
    for the wide shape): ragged seeded histories, 2 teacher-forced steps, logits, greedy ids and
    appended K/V against the oracle."""
    _say("wide batch decode B=%d %s" % (B, shape.name))
    from oracle import OracleModel, greedy
    w = synth.make_weights(shape, seed=21, gain_std=0.1)
    ctx = [int(n) for n in synth.uniform_lengths(22 + B, B, 0, 700)]
    gran = cbd.lib().cbd_slab_granule_tokens()
    arena = sum((n + 4 + gran - 1) // gran * gran for n in ctx) * shape.kv_bytes_per_token()
    eng = cbd.Engine(w, arena_bytes=arena, max_batch=64, max_prefill_tokens=64, max_position=1024)
    orc = OracleModel(w)
    ids, oids = [], []
    for r, n in enumerate(ctx):
        i = eng.alloc(n + 4)
        o = orc.new_sequence()
        if n:
            k, v = synth.kv_history(shape, 23, r, n)
            eng.append(i, to_dev_bits(torch, k), to_dev_bits(torch, v))
            orc.append_history(o, k, v)
        ids.append(i)
        oids.append(o)
    tok = synth.prompts(24, [B], shape.vocab)[0].astype(np.int64)
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    for step in range(2):
        eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits, nxt)
        ref = orc.decode_step_batch(oids, tok)
        torch.cuda.synchronize()
        errs = assert_logits_close(logits.cpu().numpy(), ref, "B=%d step %d" % (B, step))
        check_greedy(nxt.cpu().numpy(), ref, errs, "B=%d step %d" % (B, step))
        tok = greedy(ref)
    for r in (0, B // 2, B - 1):
        k, v = eng.read(ids[r], ctx[r], 2)
        torch.cuda.synchronize()
        compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[oids[r]].k)[:, ctx[r]:ctx[r] + 2], "K")
        compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[oids[r]].v)[:, ctx[r]:ctx[r] + 2], "V")
    eng.close()


def test_segmented_prefill_no_leakage_gpu(torch, cbd):
    """Changing one segment's tokens leaves the others' logits and slabs unchanged on the GPU too."""
    _say("segmented prefill leakage")
    shape = MID
    w = synth.make_weights(shape, seed=4)
    lengths = [40, 1, 77, 130, 64]
    pr = synth.prompts(13, lengths, shape.vocab)
    pr2 = [p.copy() for p in pr]
    pr2[2] = (pr2[2] + 7) % shape.vocab
    outs = []
    for prompts in (pr, pr2):
        eng = cbd.Engine(w, arena_bytes=16 * 256 * shape.kv_bytes_per_token(), max_batch=8,
                         max_prefill_tokens=512, max_position=1024)
        ids = [eng.alloc(256) for _ in lengths]
        toks = torch.from_numpy(np.concatenate(prompts).astype(np.int32)).cuda()
        lg = torch.empty((len(lengths), shape.vocab), dtype=torch.float32, device="cuda")
        eng.prefill_segmented(ids, lengths, toks, lg)
        slabs = [eng.read(i, 0, n) for i, n in zip(ids, lengths)]
        torch.cuda.synchronize()
        outs.append((lg.cpu().numpy(), [(k.cpu().numpy(), v.cpu().numpy()) for k, v in slabs]))
        eng.close()
    (l1, s1), (l2, s2) = outs
    for s in (0, 1, 3, 4):
        assert np.array_equal(l1[s], l2[s])
        assert np.array_equal(s1[s][0], s2[s][0]) and np.array_equal(s1[s][1], s2[s][1])
    assert not np.allclose(l1[2], l2[2])
    # and the prefill agrees with the oracle
    from oracle import OracleModel
    orc = OracleModel(w, cache_all_layers=True)
    oids = [orc.new_sequence() for _ in lengths]
    ref = orc.prefill_segmented(oids, pr)
    assert_logits_close(l1, ref, "prefill")
    for j, o in enumerate(oids):
        compare_slab_bits(s1[j][0], np.stack(orc.seqs[o].k), "K")


def test_chunked_prefill_continuation(torch, cbd):
    """Prefill segments that continue their sequences (chunked admission with decode steps between):
    sequence 0's prompt in chunks of 64, 50 and 36 tokens (starts at 0, 64, 114); sequence 1 prefilled,
    decoded two steps, then continued with 17 more prompt tokens (start 42); sequence 2 fresh in the
    second call. Every call's last logits, every decode step and the final slabs against the oracle."""
    _say("chunked prefill continuation")
    from oracle import OracleModel, greedy
    shape = MID
    w = synth.make_weights(shape, seed=6)
    p0, p1, p1b, p2 = synth.prompts(21, [150, 40, 17, 20], shape.vocab)
    eng = cbd.Engine(w, arena_bytes=16 * 256 * shape.kv_bytes_per_token(), max_batch=8, max_prefill_tokens=256,
                     max_position=1024)
    orc = OracleModel(w, cache_all_layers=True)
    ids = [eng.alloc(256) for _ in range(3)]
    oids = [orc.new_sequence() for _ in range(3)]

    def prefill(rows, segs, what):
        toks = torch.from_numpy(np.concatenate(segs).astype(np.int32)).cuda()
        lg = torch.empty((len(rows), shape.vocab), dtype=torch.float32, device="cuda")
        nx = torch.empty(len(rows), dtype=torch.int32, device="cuda")
        eng.prefill_segmented([ids[r] for r in rows], [len(x) for x in segs], toks, lg, nx)
        ref = orc.prefill_segmented([oids[r] for r in rows], segs)
        torch.cuda.synchronize()
        errs = assert_logits_close(lg.cpu().numpy(), ref, what)
        check_greedy(nx.cpu().numpy(), ref, errs, what)
        return greedy(ref)

    def decode(rows, toks, what):
        lg = torch.empty((len(rows), shape.vocab), dtype=torch.float32, device="cuda")
        nx = torch.empty(len(rows), dtype=torch.int32, device="cuda")
        eng.decode_step_batch([ids[r] for r in rows], torch.from_numpy(np.asarray(toks, dtype=np.int32)).cuda(), lg, nx)
        ref = orc.decode_step_batch([oids[r] for r in rows], np.asarray(toks, dtype=np.int64))
        torch.cuda.synchronize()
        errs = assert_logits_close(lg.cpu().numpy(), ref, what)
        check_greedy(nx.cpu().numpy(), ref, errs, what)
        return greedy(ref)

    t = prefill([0, 1], [p0[:64], p1], "call 1")
    t1 = decode([1], [t[1]], "decode 1")
    t = prefill([0, 2], [p0[64:114], p2], "call 2 (sequence 0 from 64, sequence 2 fresh)")
    t12 = decode([1, 2], [t1[0], t[1]], "decode 2")
    t = prefill([0, 1], [p0[114:], p1b], "call 3 (sequence 0 from 114, sequence 1 from 42)")
    decode([0, 1, 2], [t[0], t[1], t12[1]], "decode 3")
    for i, o, n in zip(ids, oids, [151, 60, 22]):
        assert eng.length(i) == n == orc.seqs[o].length
        k, v = eng.read(i, 0, n)
        torch.cuda.synchronize()
        compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[o].k), "K slab %d" % i)
        compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[o].v), "V slab %d" % i)
    # a continuation that would pass the slab's capacity is rejected without changing it
    big = torch.zeros(256, dtype=torch.int32, device="cuda")
    lg = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    with pytest.raises(cbd.CbdError) as e:
        eng.prefill_segmented([ids[0]], [106], big, lg)
    assert e.value.status == cbd.CBD_E_CAPACITY and eng.length(ids[0]) == 151
    eng.close()


def test_continuous_schedule_join_leave(torch, cbd):
    """A continuous-batching schedule through the C ABI, every call against the oracle: rows join by
    prefill (one a single token, one in two chunks while the others decode), leave between steps (a
    freed slab is handed to the next joiner with the old K/V still in it), and the batch order changes
    from step to step. Logits and greedy ids at every call, slabs bit for bit at the end."""
    _say("continuous schedule")
    from oracle import OracleModel, greedy
    shape = synth.TINY
    w = synth.make_weights(shape, seed=8, gain_std=0.1)
    eng = cbd.Engine(w, arena_bytes=4 * 256 * shape.kv_bytes_per_token(), max_batch=8, max_prefill_tokens=64,
                     max_position=1024)
    orc = OracleModel(w, cache_all_layers=True)
    pr = dict(zip("ABCDE", synth.prompts(31, [20, 7, 33, 1, 50], shape.vocab)))
    gid, oid, nxt = {}, {}, {}  # name -> GPU slab id, oracle id, next token (teacher-forced)
    done = {}

    def prefill(items, what):
        names = [n for n, _ in items]
        segs = [pr[n][lo:hi] for n, (lo, hi) in items]
        for n, (lo, hi) in items:
            if lo == 0:
                gid[n] = eng.alloc(256)
                oid[n] = orc.new_sequence()
        toks = torch.from_numpy(np.concatenate(segs).astype(np.int32)).cuda()
        lg = torch.empty((len(items), shape.vocab), dtype=torch.float32, device="cuda")
        nx = torch.empty(len(items), dtype=torch.int32, device="cuda")
        eng.prefill_segmented([gid[n] for n in names], [len(x) for x in segs], toks, lg, nx)
        ref = orc.prefill_segmented([oid[n] for n in names], segs)
        torch.cuda.synchronize()
        errs = assert_logits_close(lg.cpu().numpy(), ref, what)
        check_greedy(nx.cpu().numpy(), ref, errs, what)
        for n, t in zip(names, greedy(ref)):
            nxt[n] = int(t)

    def step(names, what):
        toks = np.array([nxt[n] for n in names])
        lg = torch.empty((len(names), shape.vocab), dtype=torch.float32, device="cuda")
        nx = torch.empty(len(names), dtype=torch.int32, device="cuda")
        eng.decode_step_batch([gid[n] for n in names], torch.from_numpy(toks.astype(np.int32)).cuda(), lg, nx)
        ref = orc.decode_step_batch([oid[n] for n in names], toks)
        torch.cuda.synchronize()
        errs = assert_logits_close(lg.cpu().numpy(), ref, what)
        check_greedy(nx.cpu().numpy(), ref, errs, what)
        for n, t in zip(names, greedy(ref)):
            nxt[n] = int(t)

    def leave(n):
        k, v = eng.read(gid[n], 0, eng.length(gid[n]))
        torch.cuda.synchronize()
        compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[oid[n]].k), "K %s" % n)
        compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[oid[n]].v), "V %s" % n)
        done[n] = eng.length(gid[n])
        eng.free(gid[n])
        orc.free_sequence(oid[n])

    prefill([("A", (0, 20)), ("B", (0, 7))], "t0 prefill A, B")
    step(["A", "B"], "t1")
    step(["B", "A"], "t2")
    leave("B")  # B's granules hold its K/V when C takes them
    prefill([("C", (0, 33))], "t3 prefill C")
    step(["C", "A"], "t3")
    prefill([("D", (0, 1))], "t4 prefill D (one token)")
    step(["A", "D", "C"], "t4")
    step(["D", "C", "A"], "t5")
    leave("A")
    prefill([("E", (0, 26))], "t6 prefill E, first chunk")
    step(["C", "D"], "t6")
    prefill([("E", (26, 50))], "t7 prefill E, second chunk")
    step(["E", "C", "D"], "t7")
    step(["D", "E", "C"], "t8")
    for n in ("C", "D", "E"):
        leave(n)
    assert done == {"A": 25, "B": 9, "C": 39, "D": 6, "E": 52}
    eng.close()


def test_int4_model_decode(torch, cbd):
    """int4-affine weights through prefill and 3 teacher-forced steps."""
    _say("int4 model")
    from oracle import OracleModel, greedy
    shape = MID_INT4
    w = synth.make_weights(shape, seed=5, gain_std=0.1)
    lengths = [9, 30, 2]
    prompts = synth.prompts(14, lengths, shape.vocab)
    eng = cbd.Engine(w, arena_bytes=16 * 256 * shape.kv_bytes_per_token(), max_batch=8, max_prefill_tokens=128,
                     max_position=1024)
    orc = OracleModel(w, cache_all_layers=True)
    ids, oids, got, gtok, ref = _prefill_both(torch, cbd, eng, orc, lengths, prompts, 64)
    errs = assert_logits_close(got, ref, "int4 prefill")
    check_greedy(gtok, ref, errs, "int4 prefill")
    tok = greedy(ref)
    logits = torch.empty((3, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(3, dtype=torch.int32, device="cuda")
    for step in range(3):
        eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), logits, nxt)
        ref = orc.decode_step_batch(oids, tok)
        torch.cuda.synchronize()
        errs = assert_logits_close(logits.cpu().numpy(), ref, "int4 step %d" % step)
        check_greedy(nxt.cpu().numpy(), ref, errs, "int4 step %d" % step)
        tok = greedy(ref)
    eng.close()


# ----------------------------------------------------------------------------- seeded top-p sampling

SAMPLE_SHAPE = synth.ModelShape("sample-v128256", 1, 256, 4, 1, 64, 512, 128256, 10000.0)


def _sample_ok(logits, temp, top_p, seed, index, got, tol=2e-6):
    """The GPU token against the oracle's selection on the same logits: equal, unless the draw or the
    nucleus edge lies within `tol` (probability mass; the kernel's exp and fixed point put its masses
    within about 1e-6 of the oracle's) of a boundary, where a neighbour in the oracle's order is
    accepted too. Returns whether the token differs from the oracle's (an accepted neighbour)."""
    from oracle import nucleus_order, sample_row, uniform_draw
    want = sample_row(logits, temp, top_p, seed, index)
    if temp == 0:
        assert got == want, "greedy row: got %d, want %d" % (got, want)
        return False
    order, p, cum, n = nucleus_order(logits, temp, top_p)
    ambiguous = set()
    if abs(cum[n - 1] - top_p) < tol or (n >= 2 and abs(cum[n - 2] - top_p) < tol):
        for nn in (n - 1, n, n + 1):  # the nucleus one token shorter or longer
            if 1 <= nn <= len(order):
                t = uniform_draw(seed, index) * cum[nn - 1]
                j = min(int(np.searchsorted(cum[:nn], t, side="right")), nn - 1)
                ambiguous.update(int(order[k]) for k in range(max(0, j - 1), min(nn, j + 2)))
    t = uniform_draw(seed, index) * cum[n - 1]
    j = min(int(np.searchsorted(cum[:n], t, side="right")), n - 1)
    if (j > 0 and abs(t - cum[j - 1]) < tol) or abs(cum[j] - t) < tol:
        ambiguous.update(int(order[k]) for k in range(max(0, j - 1), min(n, j + 2)))
    if got == want:
        return False
    assert got in ambiguous, "got %d, want %d (order position %d of nucleus %d)" % (
        got, want, int(np.where(order == got)[0][0]) if got in order else -1, n)
    return True


def test_sample_top_p_matches_oracle(torch, cbd):
    """sample_top_p over 128256-token rows: temperatures 0 (greedy), 0.5, 1, 2; top_p 1e-6 .. 1;
    random, peaked, heavily tied (logits on a 0.5 grid) and all-equal rows; every token against the
    oracle's selection on the same logits."""
    _say("sample_top_p vs oracle")
    eng = cbd.Engine(synth.make_weights(SAMPLE_SHAPE, seed=1), arena_bytes=1 << 20, max_batch=64,
                     max_prefill_tokens=64, max_position=256)
    V = SAMPLE_SHAPE.vocab
    rng = np.random.Generator(np.random.PCG64(77))
    rows = []
    for kind in range(16):
        if kind < 6:
            x = rng.normal(0.0, 2.0, V)
        elif kind < 9:
            x = rng.normal(0.0, 1.0, V)
            x[rng.integers(0, V, 5)] += 12.0  # a few dominant tokens
        elif kind < 13:
            x = np.round(rng.normal(0.0, 2.0, V) * 2.0) / 2.0  # many exact ties
        elif kind < 15:
            x = np.zeros(V)  # all tokens tied
        else:
            x = rng.normal(0.0, 4.0, V)
        rows.append(x.astype(np.float32))
    temps = [0.0, 0.5, 1.0, 2.0]
    tops = [1.0, 0.95, 0.5, 1e-6, 0.999]
    cases = []
    for i, x in enumerate(rows):
        for k in range(4):
            cases.append((x, temps[(i + k) % 4], tops[(i + 2 * k) % 5], 1000 + 7 * i + k, 3 * i + k))
    amb = 0
    for c0 in range(0, len(cases), 64):
        chunk = cases[c0:c0 + 64]
        L = torch.from_numpy(np.stack([c[0] for c in chunk])).cuda()
        out = torch.full((len(chunk),), -1, dtype=torch.int32, device="cuda")
        eng.sample_top_p(L, [c[1] for c in chunk], [c[2] for c in chunk], [c[3] for c in chunk],
                         [c[4] for c in chunk], out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for c, g in zip(chunk, got):
            amb += _sample_ok(c[0].astype(np.float64), c[1], c[2], c[3], c[4], int(g))
    _say("sample_top_p: %d cases, %d neighbours of the oracle's token at a rounding-close boundary" % (
        len(cases), amb))
    assert amb <= len(cases) // 10
    eng.close()


def test_sample_top_p_frequencies_and_draws(torch, cbd):
    """Small vocabulary (1024, a few tokens carry the mass): 4096 draws of one row with sample indices
    0..4095, each token against the oracle, and the frequencies against the probabilities."""
    _say("sample_top_p frequencies")
    shape = synth.TINY
    eng = cbd.Engine(synth.make_weights(shape, seed=2), arena_bytes=1 << 20, max_batch=64, max_prefill_tokens=64,
                     max_position=256)
    x = np.full(shape.vocab, -30.0, dtype=np.float32)
    x[[3, 17, 500, 1023]] = [1.0, 0.0, -0.5, 0.7]
    L = torch.from_numpy(np.tile(x, (64, 1))).cuda()
    got = []
    for c0 in range(0, 4096, 64):
        out = torch.empty(64, dtype=torch.int32, device="cuda")
        eng.sample_top_p(L, [1.0] * 64, [1.0] * 64, [42] * 64, list(range(c0, c0 + 64)), out)
        torch.cuda.synchronize()
        got.extend(int(v) for v in out.cpu().numpy())
    amb = sum(_sample_ok(x.astype(np.float64), 1.0, 1.0, 42, i, g) for i, g in enumerate(got))
    assert amb <= 8
    from oracle import nucleus_order
    _, p, _, _ = nucleus_order(x.astype(np.float64), 1.0, 1.0)
    freq = np.bincount(np.array(got), minlength=shape.vocab) / 4096.0
    for tok in (3, 17, 500, 1023):
        assert abs(freq[tok] - p[tok]) < 4.0 * np.sqrt(p[tok] * (1 - p[tok]) / 4096.0) + 1e-3
    # rows = 0 is a no-op; bad parameters are rejected
    eng.sample_top_p(L[:0], [], [], [], [], torch.empty(0, dtype=torch.int32, device="cuda"))
    for t, tp in ((-1.0, 0.9), (1.0, 0.0), (1.0, 1.5), (float("nan"), 0.9)):
        with pytest.raises(cbd.CbdError):
            eng.sample_top_p(L[:1], [t], [tp], [1], [0], torch.empty(1, dtype=torch.int32, device="cuda"))
    eng.close()
