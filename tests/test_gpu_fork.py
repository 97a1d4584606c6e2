"""GPU parity of sequences forked from a shared prefix (kvslab_fork) against the oracle's fork.

A fork reads the parent's whole prefix blocks from the parent's slab (decode items and prefill tiles
over two slabs) and owns a copy of the block where the prefix ends; every call is compared with the
oracle, whose fork copies the prefix."""
import sys

import numpy as np
import pytest

import synth
from gpu_common import MID, GpuStoredKV, assert_logits_close, check_greedy, compare_slab_bits

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


@pytest.mark.parametrize("kv_format", ["bf16", "affine8", "affine4"])
def test_fork_prefill_decode_and_parent_retired(torch, cbd, kv_format):
    """Parent prefilled with 90 tokens; forks at 75 (boundary block copied, holding parent keys past the
    prefix), 64 (whole blocks only) and 0; each fork prefills its own rest, then mixed decode steps with
    the parent and an unrelated row; the parent is freed while its forks keep decoding."""
    from oracle import OracleModel, dequantize_affine8, greedy
    _say("fork", kv_format)
    shape = MID
    w = synth.make_weights(shape, seed=8, gain_std=0.1)
    per_tok = cbd.kv_bytes_per_token(shape, kv_format)
    eng = cbd.Engine(w, arena_bytes=16 * 256 * per_tok, max_batch=8, max_prefill_tokens=256, max_position=1024,
                     kv_format=kv_format)
    orc = OracleModel(w, cache_all_layers=True, kv_format=kv_format)
    shared, ra, rb, rc, other = synth.prompts(31, [90, 20, 45, 7, 33], shape.vocab)
    stored = GpuStoredKV(kv_format) if kv_format != "bf16" else None
    orc.stored_override = stored

    def capture(ids, oids, t0, counts):
        if stored is not None:
            stored.capture(torch, eng, list(zip(ids, oids, t0, counts)))

    def prefill(ids, oids, segs, what):
        toks = torch.from_numpy(np.concatenate(segs).astype(np.int32)).cuda()
        lg = torch.empty((len(ids), shape.vocab), dtype=torch.float32, device="cuda")
        nx = torch.empty(len(ids), dtype=torch.int32, device="cuda")
        t0 = [eng.length(i) for i in ids]
        eng.prefill_segmented(ids, [len(x) for x in segs], toks, lg, nx)
        capture(ids, oids, t0, [len(x) for x in segs])
        ref = orc.prefill_segmented(oids, segs)
        torch.cuda.synchronize()
        errs = assert_logits_close(lg.cpu().numpy(), ref, what)
        check_greedy(nx.cpu().numpy(), ref, errs, what)
        return greedy(ref)

    def decode(ids, oids, toks, what):
        lg = torch.empty((len(ids), shape.vocab), dtype=torch.float32, device="cuda")
        nx = torch.empty(len(ids), dtype=torch.int32, device="cuda")
        t0 = [eng.length(i) for i in ids]
        eng.decode_step_batch(ids, torch.from_numpy(np.asarray(toks, dtype=np.int32)).cuda(), lg, nx)
        capture(ids, oids, t0, [1] * len(ids))
        ref = orc.decode_step_batch(oids, np.asarray(toks, dtype=np.int64))
        torch.cuda.synchronize()
        errs = assert_logits_close(lg.cpu().numpy(), ref, what)
        check_greedy(nx.cpu().numpy(), ref, errs, what)
        return greedy(ref)

    par, opar = eng.alloc(256), orc.new_sequence()
    solo, osolo = eng.alloc(256), orc.new_sequence()
    t_par, t_solo = prefill([par, solo], [opar, osolo], [shared, other], "parent")
    forks = [(eng.fork(par, P, 300), orc.fork(opar, P), P) for P in (75, 64, 0)]
    for (f, of, P) in forks:
        assert eng.length(f) == P
    t_f = prefill([f for f, _, _ in forks], [of for _, of, _ in forks], [ra, rb, np.concatenate([shared[:30], rc])],
                  "fork prefill")
    ids = [par, forks[0][0], solo, forks[1][0], forks[2][0]]
    oids = [opar, forks[0][1], osolo, forks[1][1], forks[2][1]]
    toks = [t_par, t_f[0], t_solo, t_f[1], t_f[2]]
    for step in range(2):
        toks = decode(ids, oids, toks, "step %d" % step)
    used = eng.stats()["arena_bytes_used"]
    eng.free(par)  # forks still read its prefix blocks
    orc.free_sequence(opar)
    assert eng.stats()["arena_bytes_used"] == used
    ids, oids, toks = ids[1:], oids[1:], toks[1:]
    for step in range(2, 4):
        toks = decode(ids, oids, toks, "step %d (parent freed)" % step)
    # the forks' slabs read back across the shared boundary
    for f, of in ((forks[0][0], forks[0][1]), (forks[1][0], forks[1][1])):
        n = eng.length(f)
        if kv_format == "bf16":
            k, v = eng.read(f, 0, n)
            torch.cuda.synchronize()
            compare_slab_bits(k.cpu().numpy(), np.stack(orc.seqs[of].k), "K")
            compare_slab_bits(v.cpu().numpy(), np.stack(orc.seqs[of].v), "V")
        else:
            from test_gpu_kv8 import check_appended
            codes, sb = eng.kvslab_read_q8(f, 0, n)
            torch.cuda.synchronize()
            s = orc.seqs[of]
            for w_, oc, osb in ((0, s.k, s.k_sb), (1, s.v, s.v_sb)):
                check_appended(kv_format, codes.cpu().numpy()[:, :, w_], sb.cpu().numpy()[:, :, w_], np.stack(oc),
                               np.stack(osb), "fork %s" % "KV"[w_])
    if stored is not None:
        stored.assert_consumed()
        _say("  stored forms checked %d, taken from the GPU %d" % (stored.checked, stored.replaced))
    for f, _, _ in forks:
        eng.free(f)
    eng.free(solo)
    assert eng.stats()["arena_bytes_used"] == 0
    eng.close()


def test_fork_long_prefix_decode(torch, cbd):
    """Llama-3-8B attention shape (one layer): a 9000-token parent and forks at 8999, 4500 and 2048
    decoding together with the parent (split rows with items on both slabs)."""
    from oracle import OracleModel
    _say("fork long prefix")
    shape = synth.ModelShape("fork-long", 1, 4096, 32, 8, 128, 512, 1024, 500000.0)
    w = synth.make_weights(shape, seed=9, gain_std=0.1)
    eng = cbd.Engine(w, arena_bytes=64 * 256 * shape.kv_bytes_per_token(), max_batch=8, max_position=16384)
    orc = OracleModel(w, cache_all_layers=True)
    par, opar = eng.alloc(9100), orc.new_sequence()
    k, v = synth.kv_history(shape, 50, 0, 9000)
    eng.append(par, to_dev_bits(torch, k), to_dev_bits(torch, v))
    orc.append_history(opar, k, v)
    ids, oids = [par], [opar]
    for P in (8999, 4500, 2048):
        ids.append(eng.fork(par, P, P + 64))
        oids.append(orc.fork(opar, P))
    tok = np.array([5, 17, 900, 333], dtype=np.int64)
    lg = torch.empty((len(ids), shape.vocab), dtype=torch.float32, device="cuda")
    for step in range(2):
        eng.decode_step_batch(ids, torch.from_numpy(tok.astype(np.int32)).cuda(), lg)
        ref = orc.decode_step_batch(oids, tok)
        torch.cuda.synchronize()
        assert_logits_close(lg.cpu().numpy(), ref, "step %d" % step)
        tok = (tok + 1) % shape.vocab
    eng.close()


@pytest.mark.parametrize("kv_format", ["bf16", "affine8"])
def test_fork_continuous_schedule(torch, cbd, kv_format):
    """A continuous-batching schedule whose joiners fork a 40-token shared prefix from a holder sequence:
    forks at 39 (a prompt inside the prefix), 40, 40; prompts admitted in chunks while others decode;
    rows retire between steps and their slabs go to later joiners; the holder is freed while its forks
    still decode. Every call's logits and greedy ids against the oracle (which forks the same way)."""
    from oracle import OracleModel, greedy
    _say("fork continuous schedule", kv_format)
    shape = synth.TINY
    w = synth.make_weights(shape, seed=12, gain_std=0.1)
    eng = cbd.Engine(w, arena_bytes=6 * 256 * cbd.kv_bytes_per_token(shape, kv_format), max_batch=8,
                     max_prefill_tokens=128, max_position=1024, kv_format=kv_format)
    orc = OracleModel(w, cache_all_layers=True, kv_format=kv_format)
    shared = synth.prompts(61, [40], shape.vocab)[0]
    own = dict(zip("ABCD", synth.prompts(62, [0, 25, 9, 30], shape.vocab)))
    pr = {"A": shared[:40], "B": np.concatenate([shared, own["B"]]), "C": np.concatenate([shared, own["C"]]),
          "D": np.concatenate([shared, own["D"]])}
    gid, oid, nxt, done = {}, {}, {}, {}
    stored = GpuStoredKV(kv_format) if kv_format != "bf16" else None
    orc.stored_override = stored

    def capture(names, t0, counts):
        if stored is not None:
            stored.capture(torch, eng, [(gid[n], oid[n], t, c) for n, t, c in zip(names, t0, counts)])

    def run_prefill(names, segs, what):
        toks = torch.from_numpy(np.concatenate(segs).astype(np.int32)).cuda()
        lg = torch.empty((len(names), shape.vocab), dtype=torch.float32, device="cuda")
        nx = torch.empty(len(names), dtype=torch.int32, device="cuda")
        t0 = [eng.length(gid[n]) for n in names]
        eng.prefill_segmented([gid[n] for n in names], [len(x) for x in segs], toks, lg, nx)
        capture(names, t0, [len(x) for x in segs])
        ref = orc.prefill_segmented([oid[n] for n in names], segs)
        torch.cuda.synchronize()
        errs = assert_logits_close(lg.cpu().numpy(), ref, what)
        check_greedy(nx.cpu().numpy(), ref, errs, what)
        for n, t in zip(names, greedy(ref)):
            nxt[n] = int(t)

    def join(items, what):  # (name, end of the prompt part to prefill now); a new name forks first
        names, segs = [], []
        for n, hi in items:
            if n not in gid:
                p = min(len(pr[n]) - 1, 40)
                gid[n] = eng.fork(gid["H"], p, 256)
                oid[n] = orc.fork(oid["H"], p)
            lo = eng.length(gid[n])
            names.append(n)
            segs.append(pr[n][lo:hi])
        run_prefill(names, segs, what)

    def step(names, what):
        toks = np.array([nxt[n] for n in names])
        lg = torch.empty((len(names), shape.vocab), dtype=torch.float32, device="cuda")
        nx = torch.empty(len(names), dtype=torch.int32, device="cuda")
        t0 = [eng.length(gid[n]) for n in names]
        eng.decode_step_batch([gid[n] for n in names], torch.from_numpy(toks.astype(np.int32)).cuda(), lg, nx)
        capture(names, t0, [1] * len(names))
        ref = orc.decode_step_batch([oid[n] for n in names], toks)
        torch.cuda.synchronize()
        errs = assert_logits_close(lg.cpu().numpy(), ref, what)
        check_greedy(nx.cpu().numpy(), ref, errs, what)
        for n, t in zip(names, greedy(ref)):
            nxt[n] = int(t)

    def leave(n):
        done[n] = eng.length(gid[n])
        eng.free(gid[n])
        orc.free_sequence(oid[n])

    gid["H"], oid["H"] = eng.alloc(256), orc.new_sequence()
    run_prefill(["H"], [shared], "holder")
    join([("A", 40), ("B", 52)], "t0 A (fork at 39), B first chunk")
    step(["A"], "t1")
    join([("B", 65)], "t2 B second chunk")
    step(["B", "A"], "t2")
    join([("C", 49)], "t3 C")
    step(["A", "C", "B"], "t3")
    leave("A")
    step(["C", "B"], "t4")
    join([("D", 70)], "t5 D (takes A's granules)")
    leave("H")  # forks B, C and D still read its prefix
    step(["B", "D", "C"], "t5")
    step(["D", "C", "B"], "t6")
    for n in ("B", "C", "D"):
        leave(n)
    assert done == {"A": 43, "H": 40, "B": 70, "C": 53, "D": 72}
    if stored is not None:
        stored.assert_consumed()
    assert eng.stats()["arena_bytes_used"] == 0
    eng.close()
