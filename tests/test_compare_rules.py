"""CPU checks of the comparison rules the GPU parity tests apply (no GPU).

The affine K/V rule accepts a stored form that differs from the oracle's own only where the oracle's
unrounded value lies within the projection bound of a decision boundary; these tests plant both kinds
of difference in the oracle's own forms and check that the rule tells them apart, and that the
oracle continues from an accepted form."""
import numpy as np
import pytest

import synth
from gpu_common import PROJ_ETA, GpuStoredKV, affine_decision_ok, bf16_order, compare_slab_bits
from oracle import OracleModel, f64_to_bf16_bits, round_to_bf16
from oracle.kvquant import quantize_affine


def _heads(seed, n, dh=128):
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, 1.28, size=(n, 8, dh))


@pytest.mark.parametrize("nbits", [8, 4])
def test_own_decision_is_valid(nbits):
    y = _heads(1, 300)
    codes, sb = quantize_affine(f64_to_bf16_bits(y), 64, nbits)
    assert affine_decision_ok(y, codes, sb, nbits, eta=0.0).all()
    assert affine_decision_ok(y, codes, sb, nbits).all()


@pytest.mark.parametrize("nbits", [8, 4])
def test_decisions_from_values_within_the_bound_are_valid(nbits):
    """Values moved by up to the projection bound: their decisions pass although some differ."""
    y = _heads(2, 2000)
    E = PROJ_ETA * np.max(np.abs(y), axis=-1, keepdims=True)
    moved = y + np.random.default_rng(3).uniform(-1, 1, size=y.shape) * E
    codes, sb = quantize_affine(f64_to_bf16_bits(moved), 64, nbits)
    own_codes, own_sb = quantize_affine(f64_to_bf16_bits(y), 64, nbits)
    differ = np.any(codes != own_codes, axis=-1) | np.any(sb != own_sb, axis=(-1, -2))
    assert differ.sum() > 10  # the case the rule exists for does occur
    assert affine_decision_ok(y, codes, sb, nbits).all()
    assert not affine_decision_ok(y, codes, sb, nbits, eta=0.0).all()


@pytest.mark.parametrize("nbits", [8, 4])
def test_planted_mistakes_are_rejected(nbits):
    L = (1 << nbits) - 1
    y = _heads(4, 64)
    codes, sb = quantize_affine(f64_to_bf16_bits(y), 64, nbits)
    x = round_to_bf16(y).astype(np.float32)
    q = (x.reshape(64, 8, 2, 64) - sb[..., 1:2]) / sb[..., 0:1]
    # an element far from a half-code boundary, not clamped at the top
    frac = np.abs(q - np.floor(q) - 0.5)
    idx = np.argwhere((frac > 0.2) & (np.rint(q) < L - 1))[0]
    bad = codes.copy().reshape(64, 8, 2, 64)
    bad[tuple(idx)] += 1
    assert not affine_decision_ok(y, bad.reshape(codes.shape), sb, nbits)[tuple(idx[:3])]
    for col, factor in ((0, 1.02), (1, 1.0)):  # scale off by 2%; bias off by 2% of the range
        sb2 = sb.copy()
        if col == 0:
            sb2[..., 0] *= np.float32(factor)
        else:
            sb2[..., 1] += np.float32(0.02) * sb[..., 0] * L
        assert not affine_decision_ok(y, codes, sb2, nbits).any()
    # two elements of different codes exchanged (a transposed index)
    sw = codes.copy().reshape(64, 8, 2, 64)
    g = sw[0, 0, 0]
    i, j = int(np.argmin(g)), int(np.argmax(g))
    g[i], g[j] = g[j], g[i]
    assert not affine_decision_ok(y, sw.reshape(codes.shape), sb, nbits)[0, 0, 0]
    # a constant group must carry code 0
    yc = np.full((1, 1, 64), 0.375)
    c0, s0 = quantize_affine(f64_to_bf16_bits(yc), 64, nbits)
    assert affine_decision_ok(yc, c0, s0, nbits).all()
    c1 = c0.copy()
    c1[0, 0, 5] = 1
    assert not affine_decision_ok(yc, c1, s0, nbits).any()


@pytest.mark.parametrize("fmt", ["affine8", "affine4"])
def test_stored_forms_feed_the_oracle(fmt):
    """An oracle fed another oracle's stored forms through GpuStoredKV reproduces it exactly; forms
    made from values moved within the bound are taken and carried into later layers; a form that is no
    valid decision fails."""
    shape = synth.TINY
    nbits = 8 if fmt == "affine8" else 4
    w = synth.make_weights(shape, seed=5, gain_std=0.1)
    prompt = synth.prompts(7, [9], shape.vocab)[0]
    seen = {}

    def record(sid, layer, pos, which, y, stored):
        seen[(layer, pos, which)] = np.array(y)
        return stored

    def run(override):
        o = OracleModel(w, cache_all_layers=True, kv_format=fmt)
        o.stored_override = override
        sid = o.new_sequence()
        return o.prefill(sid, prompt)

    ref_logits = run(record)
    L, n = shape.n_layers, len(prompt)

    def forms(layer0_move=None):
        """Stored forms [L, n, 2, Hkv, Dh] of the recorded values (layer 0 optionally moved)."""
        codes = np.zeros((L, n, 2, shape.n_kv_heads, shape.head_dim), np.uint8)
        sb = np.zeros((L, n, 2, shape.n_kv_heads, shape.head_dim // 64, 2), np.float32)
        for l in range(L):
            for p in range(n):
                for wi, which in enumerate("kv"):
                    y = seen[(l, p, which)]
                    if l == 0 and layer0_move is not None:
                        y = layer0_move(y)
                    codes[l, p, wi], sb[l, p, wi] = quantize_affine(f64_to_bf16_bits(y)[None], 64, nbits)
        st = GpuStoredKV(fmt)
        st.add(0, 0, codes, sb)
        return st

    st = forms()
    assert np.array_equal(run(st), ref_logits)
    st.assert_consumed()
    assert st.checked == 2 * L * n and st.replaced == 0

    # a stand-in for the GPU: an oracle whose every K/V value is moved within the bound before it is
    # rounded and quantized; a second oracle fed its forms follows it exactly, taking the moved
    # decisions as inputs
    rng = np.random.default_rng(11)
    moved = {}

    def simulated(sid, layer, pos, which, y, stored):
        E = PROJ_ETA * np.max(np.abs(y), axis=-1, keepdims=True)
        c, sbp = quantize_affine(f64_to_bf16_bits(y + rng.uniform(-1, 1, size=y.shape) * E)[None], 64, nbits)
        moved[(layer, pos, which)] = (c[0], sbp[0])
        return (c, sbp)

    sim_logits = run(simulated)
    codes = np.stack([np.stack([np.stack([moved[(l, p, x)][0] for x in "kv"]) for p in range(n)]) for l in range(L)])
    sb = np.stack([np.stack([np.stack([moved[(l, p, x)][1] for x in "kv"]) for p in range(n)]) for l in range(L)])
    st = GpuStoredKV(fmt)
    st.add(0, 0, codes, sb)
    got = run(st)
    st.assert_consumed()
    assert st.replaced > 0  # some decisions moved and were taken
    assert np.array_equal(got, sim_logits)

    def beyond(y):  # one element moved by a quarter of its group's range: a different code, not a boundary case
        y = y.copy()
        y[1, 10] += 0.25 * (y[1, :64].max() - y[1, :64].min())
        return y

    with pytest.raises(AssertionError):
        run(forms(beyond))


def test_slab_ulp_rule():
    r = synth.f32_to_bf16_bits(np.random.default_rng(0).normal(0, 1, (2, 50, 2, 64)).astype(np.float32))
    assert np.array_equal(bf16_order(np.array([0x0000, 0x8000, 0x0001, 0x8001], np.uint16)), [0, 0, 1, -1])
    compare_slab_bits(r, r)
    g = r.copy()
    g.reshape(-1)[::97] += 1  # one ulp up on about 1% of the entries: allowed
    compare_slab_bits(g, r)
    g = r.copy()
    g.reshape(-1)[::50] += 2  # two ulps on 2% of the entries: rejected
    with pytest.raises(AssertionError):
        compare_slab_bits(g, r)
