"""Helpers shared by the GPU parity tests (comparison rules, engine set-up)."""
import numpy as np

import synth

# Logit tolerance per row: max |gpu - oracle| <= 1e-2 * max |oracle|.
LOGIT_RTOL = 1e-2


def assert_logits_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite logits"
    errs = []
    for r in range(ref.shape[0]):
        err = np.max(np.abs(got[r] - ref[r]))
        bound = LOGIT_RTOL * np.max(np.abs(ref[r]))
        assert err <= bound, "%s row %d: max|dlogit| %.4g > %.4g" % (what, r, err, bound)
        errs.append(err)
    return np.array(errs)


def check_greedy(gpu_tok, ref_logits, errs, what=""):
    """Greedy ids must match wherever the oracle's top-1/top-2 margin exceeds 2x the row's error.

    Returns the number of tie-ambiguous rows (margin inside the band)."""
    ambiguous = 0
    for r in range(ref_logits.shape[0]):
        row = ref_logits[r]
        top = np.argsort(-row, kind="stable")[:2]
        orc_tok = int(top[0])
        # lowest id among exact maxima
        orc_tok = int(np.flatnonzero(row == row[orc_tok])[0])
        margin = row[top[0]] - row[top[1]]
        if margin > 2 * errs[r]:
            assert int(gpu_tok[r]) == orc_tok, "%s row %d: gpu token %d != oracle %d (margin %.3g, err %.3g)" % (
                what, r, int(gpu_tok[r]), orc_tok, margin, errs[r])
        else:
            ambiguous += 1
    return ambiguous


# Entries of a bf16 slab that must lie within one bf16 ulp of the oracle's.
SLAB_ULP_FRAC = 0.99


def bf16_order(bits):
    """bf16 bit patterns -> integers in value order, adjacent values one apart (+0 and -0 both 0)."""
    b = np.asarray(bits).view(np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def compare_slab_bits(gpu_bits, ref_bits, what=""):
    """Slab contents: values within one bf16 ulp, indexing exact.

    Values: at least SLAB_ULP_FRAC of the entries lie within one bf16 ulp of the
    oracle's (K/V come out of a projection of activations carried as bf16
    (hi, lo) pairs, about 16 significant bits, and accumulated in fp32, so a
    value the oracle computes close to a bf16 rounding boundary may round to
    the neighbouring bf16 value; near-zero entries, whose ulp is below the
    projection's absolute error, may differ by more); and per layer
    max |gpu - oracle| <= 1e-2 * max |oracle|. Indexing: every stored position
    is nearest (L2) to the oracle's vector at the same position (or ties it),
    per layer and KV head. Returns the fraction of bit-identical entries."""
    g16 = np.asarray(gpu_bits).view(np.uint16)
    r16 = np.asarray(ref_bits).view(np.uint16)
    assert g16.shape == r16.shape, (g16.shape, r16.shape)
    g = synth.bf16_bits_to_f32(g16).astype(np.float64)
    r = synth.bf16_bits_to_f32(r16).astype(np.float64)
    assert np.all(np.isfinite(g)), what + ": non-finite slab entries"
    if g16.size:
        within = float(np.mean(np.abs(bf16_order(g16) - bf16_order(r16)) <= 1))
        assert within >= SLAB_ULP_FRAC, "%s: %.4f of the entries within 1 bf16 ulp (< %.2f)" % (
            what, within, SLAB_ULP_FRAC)
    for l in range(g.shape[0]):
        err = np.max(np.abs(g[l] - r[l]))
        assert err <= LOGIT_RTOL * np.max(np.abs(r[l])), "%s layer %d: max|d| %.4g" % (what, l, err)
        n = g.shape[1]
        if n >= 2:
            for j in range(g.shape[2]):
                a, b = g[l, :, j, :], r[l, :, j, :]
                d2 = (a * a).sum(1)[:, None] - 2 * a @ b.T + (b * b).sum(1)[None, :]
                # the oracle vector of the same position is a nearest one (ties: repeated tokens give
                # identical V rows at layer 0)
                diag = d2[np.arange(n), np.arange(n)]
                assert np.all(diag <= d2.min(axis=1) + 1e-9 * (1 + np.abs(diag))), \
                    "%s layer %d head %d: slot mismatch" % (what, l, j)
    return float((g16 == r16).mean())


# shapes used only by the parity tests (random-init, small enough for the oracle)
MID = synth.ModelShape("mid-dh128-g4", 2, 512, 4, 1, 128, 1536, 2048, 500000.0)
MID_INT4 = synth.ModelShape("mid-int4", 2, 512, 4, 1, 128, 1024, 2048, 1000000.0, weight_format="int4")
# inputs of 2048 and more features: decode steps of over 32 rows split K over workgroups (gate/up;
# down with 8192 inputs, residual epilogue)
WIDE = synth.ModelShape("wide-d2048", 2, 2048, 16, 4, 128, 8192, 4096, 500000.0)


# --------------------------------------------------------------------------- affine K/V decisions

# Bound on how far the GPU's unrounded K/V value may lie from the oracle's, relative to the largest
# |value| of the same head vector. The GPU projects activations carried as bf16 (hi, lo) pairs (about
# 16 significant bits) with fp32 accumulation: its values differ from the float64 ones by about 1e-5
# of the head vector's scale; the bound keeps a margin of 25 over that.
PROJ_ETA = 2.0 ** -11


def affine_decision_ok(y, codes, sb, nbits, group=64, eta=PROJ_ETA):
    """Whether each group's stored affine form is the quantization of some bf16 vector whose unrounded
    values lie within E = eta * max|y| (over the head vector) of y.

    y: float64 [..., D] unrounded values; codes [..., D]; sb float32 [..., D/group, 2] (scale, bias).
    The quantization (bias = group minimum, scale = (maximum - bias) / L, code = the float32 rounding
    of (x - bias) / scale, clamped to 0..L; code 0 for a constant group) is monotone in every input,
    so it suffices that the bias, scale and every code lie between those reached from the lowest and
    the highest bf16 values x may take: bf16(y - E) .. bf16(y + E). With eta = 0 this is equality with
    the oracle's own decision. Returns a boolean array [..., D/group]."""
    from oracle import round_to_bf16
    levels = np.float32((1 << nbits) - 1)
    y = np.asarray(y, dtype=np.float64)
    E = eta * np.max(np.abs(y), axis=-1, keepdims=True)
    shp = y.shape[:-1] + (y.shape[-1] // group, group)
    xl = round_to_bf16(y - E).astype(np.float32).reshape(shp)
    xh = round_to_bf16(y + E).astype(np.float32).reshape(shp)
    c = np.asarray(codes).reshape(shp).astype(np.float32)
    sb = np.asarray(sb, dtype=np.float32)
    s, b = sb[..., 0], sb[..., 1]
    ok_b = (xl.min(axis=-1) <= b) & (b <= xh.min(axis=-1))
    ok_s = ((xl.max(axis=-1) - b) / levels <= s) & (s <= (xh.max(axis=-1) - b) / levels)
    pos = s > 0
    safe = np.where(pos, s, np.float32(1))[..., None]
    with np.errstate(invalid="ignore"):
        c_lo = np.clip(np.rint((xl - b[..., None]) / safe), 0, levels)
        c_hi = np.clip(np.rint((xh - b[..., None]) / safe), 0, levels)
    ok_c = np.where(pos[..., None], (c_lo <= c) & (c <= c_hi), c == 0).all(axis=-1)
    return ok_b & ok_s & ok_c


class GpuStoredKV:
    """The affine K/V forms the GPU stored for tokens it computed itself, given to the oracle as inputs.

    Several stored forms are correct for a token whose bf16 value lies next to a code boundary: the
    GPU's projection may round that value to the neighbouring bf16 value, which moves the code (one
    4-bit step is 1/15 of the group's range). Used as the oracle's ``stored_override``: each K or V
    vector the oracle computes is compared with what the GPU stored at the same sequence, layer and
    position; equal forms pass through; a different form must be a valid decision for a value within
    PROJ_ETA of the oracle's own unrounded value (affine_decision_ok), and the oracle then continues
    from the GPU's form (a slab snapshot as input), so that its later layers, steps and logits see the
    same history as the GPU. Any other difference fails the test."""

    def __init__(self, fmt):
        self.nbits = 8 if fmt == "affine8" else 4
        self.table = {}
        self.checked = 0
        self.replaced = 0

    def add(self, osid, start, codes, sb):
        """Stored forms of positions start.. of oracle sequence osid: codes [L, n, 2, Hkv, Dh] and
        pairs [L, n, 2, Hkv, Dh/64, 2] (K then V, as kvslab_read_q8 returns them)."""
        codes, sb = np.asarray(codes), np.asarray(sb, dtype=np.float32)
        for l in range(codes.shape[0]):
            for p in range(codes.shape[1]):
                for w, which in enumerate("kv"):
                    self.table[(osid, l, start + p, which)] = (codes[l, p, w][None], sb[l, p, w][None])

    def capture(self, torch, eng, pairs):
        """Read what the GPU stored: pairs of (engine sequence id, oracle sequence id, first position,
        token count)."""
        for gid, osid, start, n in pairs:
            codes, sb = eng.kvslab_read_q8(gid, start, n)
            torch.cuda.synchronize()
            self.add(osid, start, codes.cpu().numpy(), sb.cpu().numpy())

    def __call__(self, sid, layer, pos, which, y, stored):
        key = (sid, layer, pos, which)
        assert key in self.table, "no GPU stored form captured for sequence %d layer %d position %d %s" % key
        gc, gsb = self.table.pop(key)
        oc, osb = stored
        self.checked += 1
        if np.array_equal(gc, oc) and np.array_equal(gsb.view(np.uint32), np.asarray(osb, np.float32).view(np.uint32)):
            return stored
        ok = affine_decision_ok(np.asarray(y)[None], gc, gsb, self.nbits)
        assert ok.all(), "sequence %d layer %d position %d %s: stored groups %s are no valid decision" % (
            sid, layer, pos, which, np.argwhere(~ok)[:, 1:].tolist())
        self.replaced += 1
        return (gc, gsb)

    def assert_consumed(self):
        assert not self.table, "captured forms the oracle never computed: %s" % sorted(self.table)[:4]
