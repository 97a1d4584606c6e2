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


def compare_slab_bits(gpu_bits, ref_bits, what=""):
    """Slab contents: values within the logit rule, indexing exact.

    Values: per layer, max |gpu - oracle| <= 1e-2 * max |oracle| (K/V come
    out of a projection whose bf16-rounded inputs differ from the oracle's
    float64 ones by up to half a bf16 ulp, so individual entries can differ
    by a few bf16 ulps). Indexing: every stored position is nearest (L2) to
    the oracle's vector at the same position (or ties it), per layer and KV head.
    Returns the fraction of bit-identical entries."""
    g16 = np.asarray(gpu_bits).view(np.uint16)
    r16 = np.asarray(ref_bits).view(np.uint16)
    assert g16.shape == r16.shape, (g16.shape, r16.shape)
    g = synth.bf16_bits_to_f32(g16).astype(np.float64)
    r = synth.bf16_bits_to_f32(r16).astype(np.float64)
    assert np.all(np.isfinite(g)), what + ": non-finite slab entries"
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
