"""Pins of the CPU oracle against closed forms, special cases and brute force.

Each check is chosen so that a plausible mistake in the oracle (a dropped
term, a wrong sign or index, a transposed operand, a wrong position) fails
at least one of them. None of them runs the oracle against itself only.
"""
import math
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle import (OracleModel, apply_rope, attend_one_head, bf16_bits_to_f64, dequant_int4,
                    dequantize_affine8, f64_to_bf16_bits, greedy, quantize_affine4, quantize_affine8, rmsnorm,
                    round_to_bf16,
                    rope_angles, silu)
from bruteforce import BruteModel

# micro shapes: small enough for the scalar brute force, big enough to have
# GQA (2 query heads per kv head), non-square matrices and several layers
MICRO = synth.ModelShape("micro", 2, 8, 4, 2, 4, 12, 19, 10000.0, weight_std=0.4)
MICRO_INT4 = replace(MICRO, name="micro-int4", weight_format="int4", group_size=4)


# --------------------------------------------------------------------------- number formats

def test_bf16_rounding_hand_values():
    one = 1.0
    ulp = 2.0 ** -7  # bf16 spacing in [1, 2)
    assert round_to_bf16(one) == one
    assert round_to_bf16(one + ulp / 2) == one                # tie -> even (1.0)
    assert round_to_bf16(one + 3 * ulp / 2) == one + 2 * ulp  # tie -> even (k = 2)
    assert round_to_bf16(one + ulp / 2 + 1e-12) == one + ulp  # just above the tie
    assert round_to_bf16(-(one + ulp / 2 + 1e-12)) == -(one + ulp)
    assert round_to_bf16(3.0 * 2.0 ** 100) == 3.0 * 2.0 ** 100
    assert f64_to_bf16_bits(1.0) == 0x3F80 and f64_to_bf16_bits(-2.0) == 0xC000


def test_bf16_rounding_matches_independent_fp32_rne():
    """On fp32 inputs the fp64 rounding must agree with the integer bit trick."""
    x = synth.normal_f32(11, 1, (200_000,), std=3.0)
    a = f64_to_bf16_bits(x.astype(np.float64))
    b = synth.f32_to_bf16_bits(x)
    assert np.array_equal(a, b)
    assert np.array_equal(bf16_bits_to_f64(a), synth.bf16_bits_to_f32(b).astype(np.float64))


def test_bf16_rounding_is_nearest_by_brute_force():
    rng = np.random.default_rng(5)
    for x in rng.normal(size=2000) * 10.0 ** rng.integers(-6, 6, size=2000):
        r = float(round_to_bf16(x))
        b = int(f64_to_bf16_bits(x))
        for nb in (b - 1, b + 1):
            alt = float(bf16_bits_to_f64(np.uint16(nb & 0xFFFF)))
            assert abs(alt - x) >= abs(r - x)


# --------------------------------------------------------------------------- blocks

def test_rmsnorm_hand_example_and_invariant():
    y = rmsnorm([3.0, 4.0], [1.0, 1.0], 0.0)
    assert np.allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    y = rmsnorm([3.0, 4.0], [2.0, -1.0], 0.0)
    assert np.allclose(y, [6 / math.sqrt(12.5), -4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    x = np.random.default_rng(0).normal(size=(5, 64)) * 7
    y = rmsnorm(x, np.ones(64), 1e-5)
    ms = (x * x).mean(-1)
    assert np.allclose((y * y).mean(-1), ms / (ms + 1e-5), rtol=1e-12)
    # eps is added inside the root: an all-zero-but-one vector
    y = rmsnorm([1.0, 0.0, 0.0, 0.0], np.ones(4), 0.25)
    assert abs(y[0] - 1.0 / math.sqrt(0.25 + 0.25)) < 1e-15


def test_rope_closed_forms():
    t, theta = 7, 10000.0
    # Dh = 2: the single pair rotates by t radians
    assert np.allclose(apply_rope([1.0, 0.0], t, theta), [math.cos(t), math.sin(t)], atol=1e-15)
    assert np.allclose(apply_rope([0.0, 1.0], t, theta), [-math.sin(t), math.cos(t)], atol=1e-15)
    # Dh = 4: pairs (0,2) at angle t and (1,3) at angle t * theta^(-1/2)
    w = t * theta ** -0.5
    assert np.allclose(apply_rope([1.0, 0, 0, 0], t, theta), [math.cos(t), 0, math.sin(t), 0], atol=1e-15)
    assert np.allclose(apply_rope([0, 1.0, 0, 0], t, theta), [0, math.cos(w), 0, math.sin(w)], atol=1e-15)
    assert np.allclose(rope_angles(3, 8, 100.0), [3, 3 / 100 ** 0.25, 3 / 100 ** 0.5, 3 / 100 ** 0.75])


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=128), rng.normal(size=128)
    assert np.array_equal(apply_rope(q, 0, 5e5), q)
    assert abs(np.linalg.norm(apply_rope(q, 31999, 5e5)) - np.linalg.norm(q)) < 1e-10
    for t, u, d in [(5, 2, 100), (0, 9, 3000), (4000, 4000, 17)]:
        a = apply_rope(q, t, 5e5) @ apply_rope(k, u, 5e5)
        b = apply_rope(q, t + d, 5e5) @ apply_rope(k, u + d, 5e5)
        assert abs(a - b) < 1e-9 * (1 + abs(a))
    # the score genuinely depends on the offset (catches a rope that ignores t)
    assert abs(apply_rope(q, 3, 5e5) @ apply_rope(k, 0, 5e5) - q @ k) > 1e-6


def _brute_attention(q, K, V):
    dh = len(q)
    s = [sum(q[d] * K[u][d] for d in range(dh)) / math.sqrt(dh) for u in range(len(K))]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    return [sum(e[u] * V[u][d] for u in range(len(K))) / z for d in range(len(V[0]))]


@pytest.mark.parametrize("n", [1, 2, 3, 18, 65])
@pytest.mark.parametrize("dh", [1, 4, 16])
def test_attention_brute_force(n, dh):
    rng = np.random.default_rng(n * 100 + dh)
    q, K, V = rng.normal(size=dh) * 2, rng.normal(size=(n, dh)), rng.normal(size=(n, dh))
    o = attend_one_head(q, K, V)
    ref = _brute_attention(list(q), K.tolist(), V.tolist())
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    V = rng.normal(size=(6, 8))
    assert np.array_equal(attend_one_head(rng.normal(size=8), rng.normal(size=(1, 8)), V[:1]), V[0])
    K = np.tile(rng.normal(size=8), (6, 1))
    assert np.allclose(attend_one_head(rng.normal(size=8), K, V), V.mean(0), atol=1e-14)
    # a dominant key selects its value; scaling by 1/sqrt(Dh) is applied
    K = np.zeros((3, 4)); K[1] = [100, 0, 0, 0]
    assert np.allclose(attend_one_head([1.0, 0, 0, 0], K, V[:3, :4]), V[1, :4], atol=1e-20)
    K = np.zeros((2, 4)); K[0] = [2 * math.log(3.0), 0, 0, 0]
    p0 = 3.0 / 4.0  # exp(2 ln3 / sqrt(4)) = 3 against exp(0) = 1
    assert np.allclose(attend_one_head([1.0, 0, 0, 0], K, V[:2, :4]), p0 * V[0, :4] + (1 - p0) * V[1, :4])


def test_silu_closed_forms():
    assert silu(0.0) == 0.0
    assert abs(silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(silu(-2.0) - (-2.0) / (1.0 + math.exp(2.0))) < 1e-16
    assert abs(silu(40.0) - 40.0) < 1e-12 and abs(silu(-800.0)) < 1e-300


def test_greedy_lowest_id_on_ties():
    assert list(greedy([[0.0, 2.0, 2.0, 1.0], [5.0, 5.0, 5.0, 5.0], [-3.0, -1.0, -2.0, -1.0]])) == [1, 0, 1]
    x = np.random.default_rng(3).normal(size=(4, 1000))
    assert np.array_equal(greedy(x), np.argmax(x, axis=1))


def test_dequant_closed_form_and_group_index():
    codes = np.array([[0, 1, 15, 7, 3, 3, 3, 3]], dtype=np.uint8)
    scale = f64_to_bf16_bits(np.array([[0.5, 0.25]]))
    bias = f64_to_bf16_bits(np.array([[-1.0, 2.0]]))
    w = dequant_int4(codes, scale, bias, 4)
    assert np.array_equal(w, [[-1.0, -0.5, 6.5, 2.5, 2.75, 2.75, 2.75, 2.75]])
    m = synth._int4_matrix(1, 9, (16, 128), 64, 0.02)
    w = dequant_int4(m["codes"], m["scale"], m["bias"], 64)
    assert abs(w.std() - 0.02) < 0.004 and abs(w.mean()) < 0.002
    # group 1 of row 3 uses scale[3, 1]
    s = float(bf16_bits_to_f64(m["scale"][3, 1])); b = float(bf16_bits_to_f64(m["bias"][3, 1]))
    assert w[3, 64 + 5] == s * int(m["codes"][3, 64 + 5]) + b


# --------------------------------------------------------------------------- whole model vs brute force

def _run_trajectory(weights, prompts, steps, kv_group=None, rtol=1e-10, kv_bits=8):
    """Oracle: prefill each prompt, then greedy decode; brute: same tokens, one at a time.
    kv_group: affine slabs of kv_bits-bit codes with that group (None: bf16 slabs)."""
    if kv_group:
        orc = OracleModel(weights, cache_all_layers=True, kv_format="affine%d" % kv_bits, kv_group=kv_group)
    else:
        orc = OracleModel(weights, cache_all_layers=True)
    ids = [orc.new_sequence() for _ in prompts]
    lg0 = orc.prefill_segmented(ids, prompts)
    bf = BruteModel(weights, kv_group=kv_group, kv_levels=(1 << kv_bits) - 1)
    for i in ids:
        bf.add_seq(i)
    brute0 = []
    for i, p in zip(ids, prompts):
        for pos, tok in enumerate(p):
            out = bf.forward_token(i, int(tok), pos)
        brute0.append(out)
    assert np.allclose(lg0, np.array(brute0), rtol=rtol, atol=1e-12)
    toks = greedy(lg0)
    for step in range(steps):
        lg = orc.decode_step_batch(ids, toks)
        ref = [bf.forward_token(i, int(t), len(p) + step) for i, t, p in zip(ids, toks, prompts)]
        assert np.allclose(lg, np.array(ref), rtol=rtol, atol=1e-12)
        toks = greedy(lg)
    # slabs: every stored K/V entry equal to the brute force's stored values
    for i in ids:
        for l in range(weights["shape"].n_layers):
            for which in (0, 1):
                Kb = np.array([[kk for kk in ent[which]] for ent in bf.kv[i][l]])
                Ko = orc.kv_values(i, l)[which]
                if kv_group:
                    assert np.allclose(Ko, Kb, rtol=1e-12, atol=1e-12)
                else:
                    assert np.array_equal(Ko, Kb)


@pytest.mark.parametrize("gain_std", [0.0, 0.3])
def test_oracle_matches_scalar_brute_force_bf16(gain_std):
    w = synth.make_weights(MICRO, seed=4, gain_std=gain_std)
    pr = synth.prompts(40, [3, 1, 5], MICRO.vocab)
    _run_trajectory(w, pr, steps=3)


def test_oracle_matches_scalar_brute_force_int4():
    w = synth.make_weights(MICRO_INT4, seed=6)
    pr = synth.prompts(41, [4, 2], MICRO_INT4.vocab)
    _run_trajectory(w, pr, steps=2)


def test_oracle_matches_scalar_brute_force_kv8():
    """Affine 8-bit slabs: the oracle (float32 rint formula) against the brute force (nearest grid
    value by search over all 256 codes), groups of 2 dims (two groups per 4-dim head)."""
    w = synth.make_weights(MICRO, seed=8, gain_std=0.2)
    pr = synth.prompts(42, [4, 6], MICRO.vocab)
    _run_trajectory(w, pr, steps=3, kv_group=2, rtol=1e-9)


def test_oracle_matches_scalar_brute_force_kv4():
    """Affine 4-bit slabs, one group per 4-dim head (two codes strictly inside each group's range)."""
    w = synth.make_weights(MICRO, seed=9, gain_std=0.2)
    pr = synth.prompts(43, [5, 3], MICRO.vocab)
    _run_trajectory(w, pr, steps=3, kv_group=4, rtol=1e-9, kv_bits=4)


# --------------------------------------------------------------------------- shared prefixes

@pytest.mark.parametrize("kv_format", ["bf16", "affine8"])
def test_fork_equals_whole_prompt(kv_format):
    """A sequence forked from a parent's first P tokens, then given the rest of its prompt and decoded,
    gives exactly what a sequence that prefilled the whole prompt gives (causal attention: the prefix
    positions never see the tokens after them), and leaves the parent untouched."""
    w = synth.make_weights(synth.TINY, seed=3, gain_std=0.1)
    shared, tail_a, tail_b = synth.prompts(51, [37, 11, 5], synth.TINY.vocab)
    for P in (37, 32, 20):
        orc = OracleModel(w, cache_all_layers=True, kv_format=kv_format)
        par = orc.new_sequence()
        orc.prefill(par, shared)
        snap = orc.copy_state()[par]
        kid = orc.fork(par, P)
        lg_fork = orc.prefill(kid, np.concatenate([shared[P:], tail_a]))
        whole = orc.new_sequence()
        lg_whole = orc.prefill(whole, np.concatenate([shared, tail_a]))
        assert np.allclose(lg_fork, lg_whole, rtol=1e-12, atol=1e-12)
        nxt = greedy(lg_whole[None])
        both = orc.decode_step_batch([kid, whole], [nxt[0], nxt[0]])
        assert np.allclose(both[0], both[1], rtol=1e-12, atol=1e-12)
        for l in range(w["shape"].n_layers):
            assert np.array_equal(orc.seqs[par].k[l], snap.k[l])
        # a second fork of the same parent decodes independently of the first
        kid2 = orc.fork(par, P)
        lg2 = orc.prefill(kid2, np.concatenate([shared[P:], tail_b]))
        ref = OracleModel(w, cache_all_layers=True, kv_format=kv_format)
        r = ref.new_sequence()
        assert np.allclose(lg2, ref.prefill(r, np.concatenate([shared, tail_b])), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- affine 8-bit K/V

def _bf16_bits_of(values):
    bits = f64_to_bf16_bits(np.asarray(values, dtype=np.float64))
    assert np.array_equal(bf16_bits_to_f64(bits), values)  # the test values are bf16 values
    return bits


def test_affine8_exact_grid_roundtrip():
    """Values on a grid b + s*c that bf16 holds exactly come back with their codes, s and b exactly."""
    rng = np.random.default_rng(3)
    c0 = np.concatenate([[0, 255], rng.integers(0, 256, 62)])
    c1 = np.concatenate([[255, 0], rng.integers(0, 256, 62)])
    v0 = -8.0 + c0 / 16.0            # s = 1/16, b = -8
    v1 = -1.0 + c1 * 2.0 ** -7       # s = 2^-7, b = -1 (multiples of 2^-7 below 1 in magnitude)
    bits = _bf16_bits_of(np.concatenate([v0, v1]))
    codes, sb = quantize_affine8(bits)
    assert np.array_equal(codes, np.concatenate([c0, c1]).astype(np.uint8))
    assert np.array_equal(sb, np.array([[1 / 16, -8.0], [2.0 ** -7, -1.0]], dtype=np.float32))
    assert np.array_equal(dequantize_affine8(codes, sb), np.concatenate([v0, v1]))


def test_affine8_codes_are_nearest_grid_points():
    """Every code is the nearest of the 256 grid values (searched exhaustively in float64), the bias
    is the group minimum, the scale (max - min)/255 in float32, and the error at most half a step."""
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1.5, (6, 2, 128)) * np.exp(rng.normal(0, 1, (6, 2, 1)))
    bits = f64_to_bf16_bits(x)
    xv = bf16_bits_to_f64(bits).reshape(6, 2, 2, 64)
    codes, sb = quantize_affine8(bits)
    s = sb[..., 0].astype(np.float64)
    b = sb[..., 1].astype(np.float64)
    assert np.array_equal(b, xv.min(axis=-1))
    assert np.array_equal(sb[..., 0], ((xv.max(axis=-1) - xv.min(axis=-1)) / 255.0).astype(np.float32))
    grid = b[..., None, None] + s[..., None, None] * np.arange(256)  # [6, 2, 2, 1, 256]
    nearest = np.argmin(np.abs(grid - xv[..., None]), axis=-1)
    # where (x - b)/s lies within float32 rounding of a half-way point (bf16 inputs make exact
    # halves common before s is rounded), the float32 decision may take either neighbour
    quo = (xv - b[..., None]) / s[..., None]
    near_half = np.abs(quo - np.floor(quo) - 0.5) < 1e-5
    cc = codes.reshape(6, 2, 2, 64).astype(np.int64)
    assert np.array_equal(cc[~near_half], nearest[~near_half])
    assert np.all(np.abs(cc - nearest)[near_half] <= 1) and near_half.sum() < 20
    err = np.abs(dequantize_affine8(codes, sb).reshape(6, 2, 2, 64) - xv)
    assert np.all(err <= s[..., None] * (0.5 + 1e-4))
    assert np.all(codes.reshape(6, 2, 2, 64).min(axis=-1) == 0)
    assert np.all(codes.reshape(6, 2, 2, 64).max(axis=-1) == 255)


def test_affine4_grid_and_nearest_codes():
    """4-bit codes: an exact grid comes back exactly (scale (max - min)/15), and random groups take the
    nearest of the 16 grid values (either neighbour only within float32 rounding of a half)."""
    rng = np.random.default_rng(4)
    c = np.concatenate([[0, 15], rng.integers(0, 16, 62)])
    v = -2.0 + c * 0.25  # s = 1/4, b = -2: bf16 holds every value
    codes, sb = quantize_affine4(_bf16_bits_of(v))
    assert np.array_equal(codes, c.astype(np.uint8))
    assert np.array_equal(sb, np.array([[0.25, -2.0]], dtype=np.float32))
    assert np.array_equal(dequantize_affine8(codes, sb), v)
    x = f64_to_bf16_bits(rng.normal(0, 2.0, (5, 3, 128)))
    xv = bf16_bits_to_f64(x).reshape(5, 3, 2, 64)
    codes, sb = quantize_affine4(x)
    s, b = sb[..., 0].astype(np.float64), sb[..., 1].astype(np.float64)
    assert np.array_equal(sb[..., 0], ((xv.max(axis=-1) - xv.min(axis=-1)) / 15.0).astype(np.float32))
    nearest = np.argmin(np.abs(b[..., None, None] + s[..., None, None] * np.arange(16) - xv[..., None]), axis=-1)
    quo = (xv - b[..., None]) / s[..., None]
    near_half = np.abs(quo - np.floor(quo) - 0.5) < 1e-5
    cc = codes.reshape(5, 3, 2, 64).astype(np.int64)
    assert np.array_equal(cc[~near_half], nearest[~near_half]) and codes.max() == 15
    assert np.all(np.abs(cc - nearest)[near_half] <= 1)


def test_affine8_constant_group_and_group_independence():
    rng = np.random.default_rng(5)
    vals = np.concatenate([np.full(64, 0.375), rng.normal(0, 1, 64)])
    bits = f64_to_bf16_bits(vals)
    codes, sb = quantize_affine8(bits)
    assert np.all(codes[:64] == 0) and sb[0, 0] == 0.0 and sb[0, 1] == np.float32(0.375)
    assert np.array_equal(dequantize_affine8(codes, sb)[:64], bf16_bits_to_f64(bits[:64]))
    # changing the second group leaves the first group's codes and pair alone, and vice versa
    bits2 = bits.copy()
    bits2[64:] = f64_to_bf16_bits(rng.normal(0, 3, 64))
    codes2, sb2 = quantize_affine8(bits2)
    assert np.array_equal(codes2[:64], codes[:64]) and np.array_equal(sb2[0], sb[0])
    assert not np.array_equal(codes2[64:], codes[64:])
    bits3 = bits.copy()
    bits3[:64] = f64_to_bf16_bits(rng.normal(0, 1, 64))
    codes3, sb3 = quantize_affine8(bits3)
    assert np.array_equal(codes3[64:], codes[64:]) and np.array_equal(sb3[1], sb[1])


def test_affine8_model_stores_quantized_history():
    """An affine8 oracle's slab holds quantize(bits) of appended bf16 history, and its attention reads
    the dequantized values: a history already on each group's grid behaves like the bf16 slab."""
    w = synth.make_weights(synth.TINY, seed=2, gain_std=0.1)
    c = synth.TINY
    rng = np.random.default_rng(9)
    n = 40
    # history on a grid: per (layer, token, head, group) b + s*c with s = 2^-7, b = -1, codes 0..255
    codes = rng.integers(0, 256, (c.n_layers, n, c.n_kv_heads, c.head_dim))
    codes[..., 0] = 0
    codes[..., 1] = 255
    vals = -1.0 + codes * 2.0 ** -7
    kb = _bf16_bits_of(vals)
    vb = _bf16_bits_of(vals[:, ::-1])
    a = OracleModel(w, cache_all_layers=True)
    q8 = OracleModel(w, cache_all_layers=True, kv_format="affine8")
    sa, sq = a.new_sequence(), q8.new_sequence()
    a.append_history(sa, kb, vb)
    q8.append_history(sq, kb, vb)
    for l in range(c.n_layers):
        assert np.array_equal(q8.seqs[sq].k[l], codes[l].astype(np.uint8))
        assert np.array_equal(q8.kv_values(sq, l)[0], a.kv_values(sa, l)[0])
        assert np.array_equal(q8.kv_values(sq, l)[1], a.kv_values(sa, l)[1])
    # one step: identical up to the new token's quantization (a small, nonzero difference)
    la = a.decode_step_batch([sa], [5])[0]
    lq = q8.decode_step_batch([sq], [5])[0]
    d = np.max(np.abs(la - lq))
    assert 0 < d < 2e-2 * np.max(np.abs(la))
    assert q8.seqs[sq].length == n + 1 and q8.seqs[sq].k_sb[0].shape == (n + 1, c.n_kv_heads, 1, 2)


# --------------------------------------------------------------------------- the pages' invariants

def _tiny_state(seed=0, lengths=(17, 5, 33, 1)):
    w = synth.make_weights(synth.TINY, seed=seed, gain_std=0.1)
    orc = OracleModel(w, cache_all_layers=True)
    pr = synth.prompts(seed + 100, lengths, synth.TINY.vocab)
    ids = [orc.new_sequence() for _ in pr]
    lg = orc.prefill_segmented(ids, pr)
    return w, orc, ids, pr, lg


def test_batched_step_equals_solo_steps():
    """A batched step of K sequences equals K solo steps (row independence)."""
    w, orc, ids, pr, lg = _tiny_state()
    toks = greedy(lg)
    snap = orc.copy_state()
    batched = orc.decode_step_batch(ids, toks)
    for r, (sid, t) in enumerate(zip(ids, toks)):
        solo = OracleModel(w, cache_all_layers=True)
        solo.seqs = {sid: snap[sid]}
        solo_lg = solo.decode_step_batch([sid], [t])[0]
        assert np.allclose(solo_lg, batched[r], rtol=1e-12, atol=1e-12)
        for l in range(w["shape"].n_layers):
            assert np.array_equal(solo.seqs[sid].k[l], orc.seqs[sid].k[l])


def test_row_permutation():
    w, orc, ids, pr, lg = _tiny_state()
    toks = greedy(lg)
    snap = orc.copy_state()
    a = orc.decode_step_batch(ids, toks)
    orc2 = OracleModel(w, cache_all_layers=True)
    orc2.seqs = snap
    perm = [2, 0, 3, 1]
    b = orc2.decode_step_batch([ids[p] for p in perm], [toks[p] for p in perm])
    assert np.allclose(b, a[perm], rtol=1e-12, atol=1e-12)


def test_prefill_equals_sequential_decode():
    w = synth.make_weights(synth.TINY, seed=1, gain_std=0.1)
    pr = synth.prompts(7, [23], synth.TINY.vocab)[0]
    a = OracleModel(w, cache_all_layers=True)
    sa = a.new_sequence()
    la = a.prefill(sa, pr)
    b = OracleModel(w, cache_all_layers=True)
    sb = b.new_sequence()
    for tok in pr:
        lb = b.decode_step_batch([sb], [tok])[0]
    assert np.allclose(la, lb, rtol=1e-9, atol=1e-9)
    for l in range(synth.TINY.n_layers):
        ka, kb = a.seqs[sa].k[l], b.seqs[sb].k[l]
        assert ka.shape == kb.shape == (23, 2, 64)
        diff = np.abs(ka.astype(np.int32) - kb.astype(np.int32))
        assert (diff == 0).mean() >= 0.999 and diff.max() <= 1


def test_chunked_prefill_equals_whole():
    """A prompt prefilled in chunks (each continuing from the sequence's length, as a joiner admitted
    one chunk per iteration) gives the whole prompt's last logits and slab: a token's computation
    depends only on the keys at positions up to its own."""
    w = synth.make_weights(synth.TINY, seed=5, gain_std=0.1)
    pr = synth.prompts(9, [23], synth.TINY.vocab)[0]
    a = OracleModel(w, cache_all_layers=True)
    sa = a.new_sequence()
    la = a.prefill(sa, pr)
    b = OracleModel(w, cache_all_layers=True)
    sb = b.new_sequence()
    for lo, hi in ((0, 7), (7, 16), (16, 23)):
        lb = b.prefill_segmented([sb], [pr[lo:hi]])[0]
        assert b.seqs[sb].length == hi
    assert np.allclose(la, lb, rtol=1e-9, atol=1e-9)
    for l in range(synth.TINY.n_layers):
        for x, y in ((a.seqs[sa].k[l], b.seqs[sb].k[l]), (a.seqs[sa].v[l], b.seqs[sb].v[l])):
            assert x.shape == y.shape == (23, 2, 64)
            diff = np.abs(x.astype(np.int32) - y.astype(np.int32))
            assert (diff == 0).mean() >= 0.999 and diff.max() <= 1
    # a chunk's first token sees the earlier chunks: the same chunk alone on a fresh sequence differs
    c = OracleModel(w, cache_all_layers=True)
    sc = c.new_sequence()
    assert not np.allclose(c.prefill(sc, pr[16:23]), lb)


def test_no_cross_segment_leakage():
    """Changing one segment's tokens leaves every other segment's logits and slab bitwise unchanged."""
    w = synth.make_weights(synth.TINY, seed=2, gain_std=0.1)
    pr = synth.prompts(8, [9, 14, 6], synth.TINY.vocab)
    a = OracleModel(w, cache_all_layers=True)
    ia = [a.new_sequence() for _ in pr]
    la = a.prefill_segmented(ia, pr)
    pr2 = [p.copy() for p in pr]
    pr2[1] = (pr2[1] + 1) % synth.TINY.vocab
    b = OracleModel(w, cache_all_layers=True)
    ib = [b.new_sequence() for _ in pr2]
    lb = b.prefill_segmented(ib, pr2)
    assert np.array_equal(la[[0, 2]], lb[[0, 2]])
    assert not np.allclose(la[1], lb[1])
    for s in (0, 2):
        for l in range(synth.TINY.n_layers):
            assert np.array_equal(a.seqs[ia[s]].k[l], b.seqs[ib[s]].k[l])
            assert np.array_equal(a.seqs[ia[s]].v[l], b.seqs[ib[s]].v[l])


def test_decode_uses_own_position_and_history():
    """Row t_s comes from its own slab; a row attends to nothing of another row."""
    w = synth.make_weights(synth.TINY, seed=3)
    o = OracleModel(w, cache_all_layers=True)
    s0, s1 = o.new_sequence(), o.new_sequence()
    k, v = synth.kv_history(synth.TINY, 3, 0, 10)
    o.append_history(s0, k, v)
    lg = o.decode_step_batch([s0, s1], [5, 5])
    assert o.seqs[s0].length == 11 and o.seqs[s1].length == 1
    # same token at different positions with different histories gives different logits
    assert not np.allclose(lg[0], lg[1])
    # a fresh row with an empty slab equals the same row run alone
    solo = OracleModel(w, cache_all_layers=True)
    t = solo.new_sequence()
    assert np.allclose(solo.decode_step_batch([t], [5])[0], lg[1], rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        o.decode_step_batch([s0, s0], [1, 2])


# --------------------------------------------------------------------------- seeded sampling

def test_philox4x64_matches_numpy_bit_generator():
    """The oracle's Philox4x64-10 block against NumPy's Philox bit generator (which increments its
    counter before producing a block, so its block n is the function at counter n + 1)."""
    from oracle import philox4x64_10
    for key, ctr in (([0, 0], [1, 0, 0, 0]), ([0x0123456789ABCDEF, 0x1111], [7, 0, 0, 0]),
                     ([2 ** 64 - 1, 5], [2 ** 40 + 3, 9, 1, 2]), ([42, 0], [123456789, 0, 0, 0])):
        prev = list(ctr)
        prev[0] -= 1
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(prev, dtype=np.uint64))
        assert [int(x) for x in bg.random_raw(4)] == philox4x64_10(ctr, key)


def test_uniform_draw_range_bits_and_moments():
    from oracle import uniform_draw
    u = np.array([uniform_draw(9, i) for i in range(20000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert np.array_equal(u * 2 ** 24, np.floor(u * 2 ** 24))  # 24 bits, exact in float32
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1.0 / 12.0) < 0.005
    # distinct seeds and indices give distinct streams
    assert uniform_draw(1, 0) != uniform_draw(2, 0) and uniform_draw(1, 0) != uniform_draw(1, 1)


def test_nucleus_closed_forms():
    """Probabilities 1/2, 1/4, 1/8, 1/8 (ids 0, 1, 2, 3; the tie ordered by id): nucleus sizes for
    several p away from the cumulative steps, and temperature 2 giving p proportional to sqrt(p)."""
    from oracle import nucleus_order
    x = np.log(np.array([0.5, 0.25, 0.125, 0.125]))
    for top_p, n_want in ((1e-9, 1), (0.45, 1), (0.6, 2), (0.8, 3), (0.9, 4), (1.0, 4)):
        order, p, cum, n = nucleus_order(x, 1.0, top_p)
        assert list(order) == [0, 1, 2, 3] and n == n_want
        assert np.allclose(p, [0.5, 0.25, 0.125, 0.125], rtol=1e-12)
    _, p2, _, _ = nucleus_order(x, 2.0, 1.0)
    q = np.sqrt([0.5, 0.25, 0.125, 0.125])
    assert np.allclose(p2, q / q.sum(), rtol=1e-12)
    # ties ordered by id whatever their position in the row
    order, _, _, _ = nucleus_order(np.log(np.array([0.125, 0.25, 0.125, 0.5])), 1.0, 1.0)
    assert list(order) == [3, 1, 0, 2]


def test_sample_row_inverse_cdf_thresholds():
    """With probabilities 1/2, 1/4, 1/8, 1/8 and the whole vocabulary: token 0 for u < 1/2, 1 for
    u < 3/4, 2 for u < 7/8, else 3; with top_p = 0.6 (nucleus {0, 1}, mass 3/4): token 0 for
    u < 2/3, else 1; greedy at temperature 0 and a vanishing top_p give the lowest-id maximum."""
    from oracle import sample_row, uniform_draw
    x = np.log(np.array([0.5, 0.25, 0.125, 0.125]))
    for i in range(400):
        u = uniform_draw(5, i)
        assert sample_row(x, 1.0, 1.0, 5, i) == (0 if u < 0.5 else 1 if u < 0.75 else 2 if u < 0.875 else 3)
        assert sample_row(x, 1.0, 0.6, 5, i) == (0 if u < 2.0 / 3.0 else 1)
    y = np.array([1.0, 3.0, -2.0, 3.0])
    assert sample_row(y, 0.0, 1.0, 1, 1) == 1
    assert all(sample_row(y, 1.0, 1e-9, s, 0) == 1 for s in range(20))


def test_sampling_frequencies_follow_the_softmax():
    from oracle import nucleus_order, sample_row
    x = np.array([0.3, -1.0, 2.0, 0.0, 1.2])
    n = 20000
    got = np.bincount([sample_row(x, 0.7, 1.0, 11, i) for i in range(n)], minlength=5) / n
    _, p, _, _ = nucleus_order(x, 0.7, 1.0)
    assert np.allclose(p, np.exp(x / 0.7) / np.exp(x / 0.7).sum(), rtol=1e-12)
    assert np.all(np.abs(got - p) < 4 * np.sqrt(p * (1 - p) / n) + 1e-3)
