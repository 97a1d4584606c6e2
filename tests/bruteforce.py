"""Scalar brute-force decoder used only to pin the oracle on micro shapes.

Written independently of ``oracle/``: plain Python floats, explicit index
loops and the ``math`` module, no numpy linear algebra. Matrices are read as
W[out][in] with y[i] = sum_j W[i][j] x[j]. Attention builds every score with
an explicit causal test instead of slicing.
"""
import math
import struct


def bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def bf16_round(x):
    """Nearest bf16 value (ties to even) by scanning the two neighbours in fp32 bit space."""
    if x == 0.0:
        return 0.0
    f = struct.unpack("<I", struct.pack("<f", x))[0]  # fp32 nearest (values here are already fp64)
    # candidates: truncations around x in bf16 space, compared in exact float arithmetic
    hi = f >> 16
    cands = [bf16_value(hi), bf16_value(hi + 1), bf16_value(hi - 1)]
    best = None
    for c in cands:
        d = abs(c - x)
        if best is None or d < best[0] or (d == best[0] and (int(_bits(c)) & 1) == 0):
            best = (d, c)
    return best[1]


def _bits(v):
    return struct.unpack("<I", struct.pack("<f", v))[0] >> 16


def mat(bits_2d):
    return [[bf16_value(b) for b in row] for row in bits_2d]


def vec(bits_1d):
    return [bf16_value(b) for b in bits_1d]


def int4_mat(m, group):
    codes, scale, bias = m["codes"], m["scale"], m["bias"]
    out = []
    for n in range(codes.shape[0]):
        row = []
        for k in range(codes.shape[1]):
            s = bf16_value(scale[n][k // group])
            b = bf16_value(bias[n][k // group])
            row.append(s * int(codes[n][k]) + b)
        out.append(row)
    return out


def matvec(W, x):
    return [sum(W[i][j] * x[j] for j in range(len(x))) for i in range(len(W))]


def norm(x, g, eps):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[i] * r * g[i] for i in range(len(x))]


def rope(x, t, theta):
    n = len(x)
    half = n // 2
    out = [0.0] * n
    for i in range(half):
        ang = t * theta ** (-(2.0 * i) / n)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = x[i] * c - x[i + half] * s
        out[i + half] = x[i + half] * c + x[i] * s
    return out


def f32_round(x):
    """Nearest float32 value of a Python float."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def affine_nearest(xs, group, levels=255):
    """Affine storage by direct search: per group, bias = min, scale = float32((max - min) / levels),
    and each element takes the code 0..levels whose grid value bias + scale * code is nearest to it
    (the lower code on an exact tie is never needed for random inputs). Returns dequantized values."""
    out = []
    for g0 in range(0, len(xs), group):
        grp = xs[g0:g0 + group]
        lo, hi = min(grp), max(grp)
        s = f32_round((hi - lo) / float(levels))
        for x in grp:
            if s == 0.0:
                out.append(lo)
                continue
            best = min(range(levels + 1), key=lambda c: abs(lo + s * c - x))
            out.append(lo + s * best)
    return out


class BruteModel:
    def __init__(self, weights, kv_group=None, kv_levels=255):
        self.kv_group = kv_group  # None: bf16 slabs; else affine slabs with this group and code range
        self.kv_levels = kv_levels
        self.cfg = cfg = weights["shape"]
        if cfg.weight_format == "int4":
            conv = lambda m: int4_mat(m, cfg.group_size)
        else:
            conv = mat
        self.E = mat(weights["embed"])
        self.LM = conv(weights["lm_head"])
        self.gout = vec(weights["final_norm"])
        self.layers = []
        for lw in weights["layers"]:
            self.layers.append({k: (vec(v) if k.endswith("norm") else conv(v)) for k, v in lw.items()})
        # kv[seq][layer] = list of (k_heads, v_heads), each a list of Hkv lists of Dh floats
        self.kv = {}

    def add_seq(self, sid):
        self.kv[sid] = [[] for _ in self.layers]

    def forward_token(self, sid, tok, pos):
        c = self.cfg
        dh, hq, hkv = c.head_dim, c.n_heads, c.n_kv_heads
        h = list(self.E[tok])
        for l, L in enumerate(self.layers):
            a = norm(h, L["attn_norm"], c.rms_eps)
            q = matvec(L["wq"], a)
            k = matvec(L["wk"], a)
            v = matvec(L["wv"], a)
            ks = [[bf16_round(z) for z in rope(k[j * dh:(j + 1) * dh], pos, c.rope_theta)] for j in range(hkv)]
            vs = [[bf16_round(z) for z in v[j * dh:(j + 1) * dh]] for j in range(hkv)]
            if self.kv_group:
                ks = [affine_nearest(x, self.kv_group, self.kv_levels) for x in ks]
                vs = [affine_nearest(x, self.kv_group, self.kv_levels) for x in vs]
            slab = self.kv[sid][l]
            assert len(slab) == pos
            slab.append((ks, vs))
            o = []
            for hh in range(hq):
                j = hh * hkv // hq
                qh = rope(q[hh * dh:(hh + 1) * dh], pos, c.rope_theta)
                scores = []
                for u in range(len(slab)):
                    if u <= pos:  # causal: own history up to and including the new token
                        scores.append(sum(qh[d] * slab[u][0][j][d] for d in range(dh)) / math.sqrt(dh))
                mx = max(scores)
                e = [math.exp(s - mx) for s in scores]
                z = sum(e)
                for d in range(dh):
                    o.append(sum(e[u] / z * slab[u][1][j][d] for u in range(len(scores))))
            y = matvec(L["wo"], o)
            h = [h[i] + y[i] for i in range(len(h))]
            b = norm(h, L["ffn_norm"], c.rms_eps)
            gt = matvec(L["w_gate"], b)
            up = matvec(L["w_up"], b)
            m = [gt[i] / (1.0 + math.exp(-gt[i])) * up[i] for i in range(len(gt))]
            y = matvec(L["w_down"], m)
            h = [h[i] + y[i] for i in range(len(h))]
        x = norm(h, self.gout, c.rms_eps)
        return matvec(self.LM, x)
