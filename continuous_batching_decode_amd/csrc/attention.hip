// Ragged per-sequence attention over persistent slabs.
//
// Page "Continuous Decode Batching - the transformer capture", section
// "decode_step_batch - paint-by-numbers": each query row rotates q and k at
// its own position t_s (delta 1), writes its new K/V into its own slab at
// t_s (delta 2), and attends only to [0..=t_s] of that slab (delta 3). The
// segmented prefill (section "REVISED") attends a token at segment-local
// position p to [0..=p] of its own segment's slab, so no query ever reads
// another sequence's keys (block-diagonal causal).
//
// Decode (decode_attention_kernel): one wave = one work item (query row, key
// range) x one KV head, for the G = Hq/Hkv query heads sharing that KV head
// (GQA: every K/V byte is read once for all of them). Keys stream straight
// from HBM in blocks of 32 in the slab's MFMA fragment layout, the next block
// in flight while the current one is used:
//   S^T[32 keys x 16 cols] = K[32 x Dh] . Q^T[Dh x 16]   (cols = heads, G used)
//   O^T[Dh x 16]          += V^T[Dh x 32] . P^T[32 x 16]
// q and p enter the products as bf16 hi + lo pairs (about 16 significant
// bits, as the activations of the weight-streaming products do); the running
// (max, sum) softmax is fp32 and per column, so rescaling never leaves the
// lane. The new token's key and value are rotated and rounded in registers,
// taken as the first key, and stored to the slab. Long histories are split
// over several items (flash-decoding); the last wave of a (row, KV head) to
// finish merges the splits with the log-sum-exp rule in a fixed order.
//
// Prefill (prefill_attention_kernel): the same products with the 16 columns
// holding 16 consecutive query tokens of one segment and one query head; each
// column masks keys after its own position (causal) and reads only its own
// segment's slab (block-diagonal). The tokens' K/V were appended beforehand.
#include "common.h"
#include "kernels.h"

namespace cbd {

namespace {

CBD_DEVICE void store_split(uint16_t* hi, uint16_t* lo, float v) {
  const uint32_t h = f32_to_bf16(v);
  *hi = (uint16_t)h;
  *lo = (uint16_t)f32_to_bf16(v - bf16_to_f32(h));
}

// 8 fp32 values -> bf16 hi and lo operands (v ~ hi + lo)
CBD_DEVICE void split8(const float (&v)[8], bf16x8_t& hi, bf16x8_t& lo) {
  u32x4_t h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    l[i] = pack_bf16x2(v[2 * i] - bf16_to_f32(h[i] & 0xFFFFu), v[2 * i + 1] - bf16_to_f32(h[i] >> 16));
  }
  hi = as_frag(h);
  lo = as_frag(l);
}

// 4 fp32 -> 4 bf16 hi values and 4 lo values, as two 8-byte words
CBD_DEVICE void split4(const float (&v)[4], uint2& hi, uint2& lo) {
  hi = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  lo = uint2{pack_bf16x2(v[0] - bf16_to_f32(hi.x & 0xFFFFu), v[1] - bf16_to_f32(hi.x >> 16)),
             pack_bf16x2(v[2] - bf16_to_f32(hi.y & 0xFFFFu), v[3] - bf16_to_f32(hi.y >> 16))};
}

CBD_DEVICE float exp_or_zero(float x, float m) { return x == -INFINITY ? 0.f : __expf(x - m); }

CBD_DEVICE void load8(const float* p, float (&x)[8]) {
  const float4 x0 = *reinterpret_cast<const float4*>(p);
  const float4 x1 = *reinterpret_cast<const float4*>(p + 4);
  x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
  x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
}

// Keys of one (slab, layer, KV head) region, streamed in blocks of 32 (K then V fragments).
template <int DH>
struct KVStream {
  static constexpr int NU = DH / 32;  // dim chunks of 32 (K fragments per 16 keys)
  static constexpr int NT = DH / 16;  // dim tiles of 16 (V fragments per 32 keys)
  const uint16_t* kbase;
  const uint16_t* vbase;
  int lane;
  CBD_DEVICE void load_k(u32x4_t (&K)[2 * NU], int b) const {
    const uint16_t* p = kbase + (int64_t)b * 32 * DH + 8 * lane;
#pragma unroll
    for (int i = 0; i < 2 * NU; ++i) K[i] = load_stream(p + 512 * i);
  }
  CBD_DEVICE void load_v(u32x4_t (&V)[NT], int b) const {
    const uint16_t* p = vbase + (int64_t)b * 32 * DH + 8 * lane;
#pragma unroll
    for (int t = 0; t < NT; ++t) V[t] = load_stream(p + 512 * t);
  }
};

// Running softmax state of the lane's column (equal in the column's 4 lanes) and its O^T tiles.
template <int DH>
struct Online {
  f32x4_t o[DH / 16];
  float m, l;
  CBD_DEVICE void clear() {
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }
};

// S^T of one block: lane holds keys 32b + 4g + e (s0) and 32b + 16 + 4g + e (s1) of its column.
template <int DH>
CBD_DEVICE void block_scores(const u32x4_t (&K)[DH / 16], const bf16x8_t (&qh)[DH / 32],
                             const bf16x8_t (&ql)[DH / 32], f32x4_t& s0, f32x4_t& s1) {
  constexpr int NU = DH / 32;
  s0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
  s1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    s0 = mfma(as_frag(K[u]), qh[u], s0);
    s0 = mfma(as_frag(K[u]), ql[u], s0);
    s1 = mfma(as_frag(K[NU + u]), qh[u], s1);
    s1 = mfma(as_frag(K[NU + u]), ql[u], s1);
  }
}

// Online softmax over block b (keys at or past lim, the limit of the lane's column, are masked),
// then O^T += V^T P^T, where P^T element i of lane group g is key kk = 8g + i of the block's V order.
template <int DH>
CBD_DEVICE void block_accumulate(const u32x4_t (&V)[DH / 16], const f32x4_t& s0, const f32x4_t& s1, int b, int g,
                                 int lim, float scale, Online<DH>& st) {
  float sv[8];
  const int k0 = 32 * b + 4 * g;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sv[e] = k0 + e < lim ? s0[e] * scale : -INFINITY;
    sv[4 + e] = k0 + 16 + e < lim ? s1[e] * scale : -INFINITY;
  }
  float bm = sv[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) bm = fmaxf(bm, sv[i]);
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  const float m_new = fmaxf(st.m, bm);
  const float alpha = exp_or_zero(st.m, m_new);
  float p[8], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = exp_or_zero(sv[i], m_new);
    ps += p[i];
  }
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  st.l = st.l * alpha + ps;
  st.m = m_new;
  bf16x8_t ph, pl;
  split8(p, ph, pl);
#pragma unroll
  for (int t = 0; t < DH / 16; ++t) {
    st.o[t] = st.o[t] * alpha;
    st.o[t] = mfma(as_frag(V[t]), ph, st.o[t]);
    st.o[t] = mfma(as_frag(V[t]), pl, st.o[t]);
  }
}

// Blocks [b_first, b_end), K0/V0 already holding block b_first. One block in registers,
// staggered: the next K loads during the softmax and P.V of this block, the next V during the next
// block's scores. The loads are unconditional (a branch around them makes the compiler's completion
// waits cover everything) and scheduling barriers keep them in this order; the last block is peeled.
template <int DH>
CBD_DEVICE void stream_blocks(const KVStream<DH>& kv, u32x4_t (&K0)[DH / 16], u32x4_t (&V0)[DH / 16], int b_first,
                              int b_end, int g, int lim, float scale, const bf16x8_t (&qh)[DH / 32],
                              const bf16x8_t (&ql)[DH / 32], Online<DH>& st) {
  for (int b = b_first; b + 1 < b_end; ++b) {
    f32x4_t s0, s1;
    block_scores<DH>(K0, qh, ql, s0, s1);
    __builtin_amdgcn_sched_barrier(0);
    kv.load_k(K0, b + 1);
    __builtin_amdgcn_sched_barrier(0);
    block_accumulate<DH>(V0, s0, s1, b, g, lim, scale, st);
    __builtin_amdgcn_sched_barrier(0);
    kv.load_v(V0, b + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (b_first < b_end) {
    f32x4_t s0, s1;
    block_scores<DH>(K0, qh, ql, s0, s1);
    block_accumulate<DH>(V0, s0, s1, b_end - 1, g, lim, scale, st);
  }
}

// Online softmax over the 64 keys of blocks b and b + 1 at once (one max, one rescale), then
// O^T += V0^T P0^T + V1^T P1^T. Same element order as block_accumulate, block by block.
template <int DH>
CBD_DEVICE void pair_accumulate(const u32x4_t (&V0)[DH / 16], const u32x4_t (&V1)[DH / 16], const f32x4_t (&s)[4],
                                int b, int g, int lim, float scale, Online<DH>& st) {
  float sv[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k0 = 32 * (b + h) + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[8 * h + e] = k0 + e < lim ? s[2 * h][e] * scale : -INFINITY;
      sv[8 * h + 4 + e] = k0 + 16 + e < lim ? s[2 * h + 1][e] * scale : -INFINITY;
    }
  }
  float bm = sv[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) bm = fmaxf(bm, sv[i]);
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  const float m_new = fmaxf(st.m, bm);
  const float alpha = exp_or_zero(st.m, m_new);
  float p0[8], p1[8], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p0[i] = exp_or_zero(sv[i], m_new);
    p1[i] = exp_or_zero(sv[8 + i], m_new);
    ps += p0[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) ps += p1[i];
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  st.l = st.l * alpha + ps;
  st.m = m_new;
  bf16x8_t ph0, pl0, ph1, pl1;
  split8(p0, ph0, pl0);
  split8(p1, ph1, pl1);
#pragma unroll
  for (int t = 0; t < DH / 16; ++t) {
    st.o[t] = st.o[t] * alpha;
    st.o[t] = mfma(as_frag(V0[t]), ph0, st.o[t]);
    st.o[t] = mfma(as_frag(V0[t]), pl0, st.o[t]);
    st.o[t] = mfma(as_frag(V1[t]), ph1, st.o[t]);
    st.o[t] = mfma(as_frag(V1[t]), pl1, st.o[t]);
  }
}

// Blocks [b_first, b_end) two at a time with two blocks in flight: (K0, V0) and (K1, V1) hold
// blocks b and b + 1 on entry (indices past the last clamp to it, so every load stays
// unconditional) and are refilled with b + 2 and b + 3 as soon as they have been used.
template <int DH>
CBD_DEVICE void stream_pairs(const KVStream<DH>& kv, u32x4_t (&K0)[DH / 16], u32x4_t (&V0)[DH / 16],
                             u32x4_t (&K1)[DH / 16], u32x4_t (&V1)[DH / 16], int b_first, int b_end, int g, int lim,
                             float scale, const bf16x8_t (&qh)[DH / 32], const bf16x8_t (&ql)[DH / 32],
                             Online<DH>& st) {
  const int last = b_end - 1;
  int b = b_first;
  f32x4_t s[4];
  for (; b + 2 < b_end; b += 2) {
    block_scores<DH>(K0, qh, ql, s[0], s[1]);
    block_scores<DH>(K1, qh, ql, s[2], s[3]);
    __builtin_amdgcn_sched_barrier(0);
    kv.load_k(K0, b + 2);
    kv.load_k(K1, min(b + 3, last));
    __builtin_amdgcn_sched_barrier(0);
    pair_accumulate<DH>(V0, V1, s, b, g, lim, scale, st);
    __builtin_amdgcn_sched_barrier(0);
    kv.load_v(V0, b + 2);
    kv.load_v(V1, min(b + 3, last));
    __builtin_amdgcn_sched_barrier(0);
  }
  if (b + 1 < b_end) {  // a last pair
    block_scores<DH>(K0, qh, ql, s[0], s[1]);
    block_scores<DH>(K1, qh, ql, s[2], s[3]);
    pair_accumulate<DH>(V0, V1, s, b, g, lim, scale, st);
  } else if (b < b_end) {  // a last single block
    block_scores<DH>(K0, qh, ql, s[0], s[1]);
    block_accumulate<DH>(V0, s[0], s[1], b, g, lim, scale, st);
  }
}

// The lane's O^T tiles (dims 16t + 4g + e of its column), times inv, to the hi/lo planes of `row`.
template <int DH>
CBD_DEVICE void store_out(const AttnArgs& a, int row, int head, int g, const f32x4_t (&o)[DH / 16], float inv) {
#pragma unroll
  for (int t = 0; t < DH / 16; ++t) {
    const float y[4] = {o[t][0] * inv, o[t][1] * inv, o[t][2] * inv, o[t][3] * inv};
    uint2 hi, lo;
    split4(y, hi, lo);
    const int64_t off = xfrag_off(row, head * DH + 16 * t + 4 * g, a.ld_out);
    *reinterpret_cast<uint2*>(a.out + off) = hi;
    *reinterpret_cast<uint2*>(a.out + a.out_plane + off) = lo;
  }
}

// An item is the same for the whole wave: keep it in scalar registers (uniform branches).
CBD_DEVICE AttnItem uniform_item(const AttnItem* items, int i) {
  AttnItem it = items[i];
  it.slab_off = ((int64_t)__builtin_amdgcn_readfirstlane((int32_t)(it.slab_off >> 32)) << 32) |
                (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)it.slab_off);
  it.stride = __builtin_amdgcn_readfirstlane(it.stride);
  it.pos = __builtin_amdgcn_readfirstlane(it.pos);
  it.row = __builtin_amdgcn_readfirstlane(it.row);
  it.k_begin = __builtin_amdgcn_readfirstlane(it.k_begin);
  it.k_end = __builtin_amdgcn_readfirstlane(it.k_end);
  it.part = __builtin_amdgcn_readfirstlane(it.part);
  it.pre_off = ((int64_t)__builtin_amdgcn_readfirstlane((int32_t)(it.pre_off >> 32)) << 32) |
               (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)it.pre_off);
  it.pre_stride = __builtin_amdgcn_readfirstlane(it.pre_stride);
  it.pre_end = __builtin_amdgcn_readfirstlane(it.pre_end);
  return it;
}

}  // namespace

// The end of a decode item: an unsplit item writes its rows; a split item publishes its unnormalised
// partial and (max, sum), and the last wave of the (row, KV head) to arrive merges the splits.
template <int DH, int G>
CBD_DEVICE void decode_finish(const AttnArgs& a, const AttnItem& it, int j, int2 rp, int lane, const Online<DH>& st) {
  constexpr int NT = DH / 16;
  const int g = lane >> 4, c16 = lane & 15;
  const f32x4_t(&o)[NT] = st.o;
  const float m_run = st.m, l_run = st.l;

  if (it.part < 0) {  // output: lane (c16 < G) holds dims 16t + 4g + e of head j*G + c16
    if (c16 < G) store_out<DH>(a, it.row, j * G + c16, g, o, 1.0f / l_run);
    return;
  }
  // split item: publish the unnormalised partial and (max, sum); the last wave of the (row, KV head)
  // merges. Partials and the arrival counter use agent-scope accesses (coherent across the XCDs'
  // L2 caches), partials 16 bytes at a time; the wave's stores are acknowledged (vmcnt 0) before its
  // arrival is counted.
  if (c16 < G) {
    const int64_t slot = (int64_t)it.part * a.n_heads + j * G + c16;
#pragma unroll
    for (int t = 0; t < NT; ++t) store_agent_x4(a.part_o, (int)((slot * DH + 16 * t + 4 * g) * 4), o[t]);
    if (g == 0) store_agent_x2(a.part_ml, (int)(slot * 2 * 4), float2{m_run, l_run});
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  int32_t* counter = a.counters + (int64_t)it.row * a.n_kv_heads + j;
  int last = 0;
  if (lane == 0) last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == rp.y - 1;
  last = __shfl(last, 0, 64);
  if (!last) return;

  // Merge with the whole wave (at most 64 splits). Lane s loads split s's (max, sum) for every head;
  // the per-head maximum and weighted sum come from wave reductions. Lane l combines output
  // elements NE*l .. NE*l + NE - 1 of the G x Dh block over the splits in order, the loads of SB
  // splits in flight at a time; the first SB are requested with the (max, sum) pairs, so up to SB
  // splits cost one memory latency.
  constexpr int NE = G * DH / 64;  // 8, 4 or 2 floats per lane
  const int ns = rp.y;
  // lane s: (max, sum) of split s for the G heads, 2G consecutive floats
  float mv[G], wv[G], Mh[G], Lh[G];
  float ml[2 * G];
  {
    const int off = (int)((((int64_t)(rp.x + min(lane, ns - 1)) * a.n_heads + j * G) * 2) * 4);
    if constexpr (G == 1) {
      const float2 x = load_agent_x2(a.part_ml, off);
      ml[0] = x.x;
      ml[1] = x.y;
    } else {
#pragma unroll
      for (int q = 0; q < G / 2; ++q) {
        const f32x4_t x = load_agent_x4(a.part_ml, off + 16 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) ml[4 * q + e] = x[e];
      }
    }
  }
  const int e0 = lane * NE, hh = e0 / DH, d0 = e0 % DH;
  const int64_t split_stride = (int64_t)a.n_heads * DH;
  const int64_t o_base = (int64_t)rp.x * a.n_heads + j * G + hh;  // slot row of split 0, in DH units
  constexpr int SB = NE >= 4 ? 8 : 16;  // registers: SB x NE floats
  float ov[SB][NE];
  auto load_batch = [&](int s0) {  // splits past the last reload it (their weight is 0)
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int off = (int)(((o_base * DH + d0) + (int64_t)min(s0 + u, ns - 1) * split_stride) * 4);
      if constexpr (NE == 2) {
        const float2 x = load_agent_x2(a.part_o, off);
        ov[u][0] = x.x;
        ov[u][1] = x.y;
      } else {
#pragma unroll
        for (int q = 0; q < NE / 4; ++q) {
          const f32x4_t x = load_agent_x4(a.part_o, off + 16 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[u][4 * q + e] = x[e];
        }
      }
    }
  };
  load_batch(0);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mv[h] = lane < ns ? ml[2 * h] : -INFINITY;  // lanes past the last split take no part
    wv[h] = lane < ns ? ml[2 * h + 1] : 0.f;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    Mh[h] = wave_max(mv[h]);
    Lh[h] = wave_sum(exp_or_zero(mv[h], Mh[h]) * wv[h]);
    wv[h] = exp_or_zero(mv[h], Mh[h]);  // lane s: weight of split s for head h
  }
  float acc[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += SB) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      float wgt = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float x = __shfl(wv[h], s0 + u, 64);
        if (hh == h) wgt = x;
      }
#pragma unroll
      for (int i = 0; i < NE; ++i) acc[i] += wgt * ov[u][i];
    }
    if (s0 + SB < ns) load_batch(s0 + SB);
  }
  float L = Lh[0];
#pragma unroll
  for (int h = 1; h < G; ++h)
    if (hh == h) L = Lh[h];
  const float inv = 1.0f / L;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int64_t off = xfrag_off(it.row, (j * G + hh) * DH + d0 + i, a.ld_out);
    store_split(a.out + off, a.out + a.out_plane + off, acc[i] * inv);
  }
  if (lane == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ============================================================================ decode

// Workgroups of CBD_ATTN_WG_WAVES waves (the waves share nothing): single-wave workgroups let the
// dispatcher spread a step's waves evenly over the compute units.
#ifndef CBD_ATTN_WG_WAVES
#define CBD_ATTN_WG_WAVES 1
#endif
constexpr int kAttnWgWaves = CBD_ATTN_WG_WAVES;
#ifndef CBD_ATTN_PD
#define CBD_ATTN_PD 2
#endif

template <int DH, int G, int PD>
__global__ __launch_bounds__(64 * kAttnWgWaves, 2) void decode_attention_kernel(AttnArgs a, int n_waves) {
  constexpr int NU = DH / 32;  // dim chunks of 32 (K fragments per 16 keys)
  constexpr int NT = DH / 16;  // dim tiles of 16 (V fragments per 32 keys)
  constexpr int PAIR = DH / 64;  // RoPE partner of chunk u is u ^ PAIR (dims d and d + Dh/2)
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kAttnWgWaves + (threadIdx.x >> 6));
  if (w >= n_waves) return;
  const int j = w % a.n_kv_heads;
  const AttnItem it = uniform_item(a.items, w / a.n_kv_heads);
  const int pos = it.pos;
  const int64_t region = (int64_t)it.stride * DH;
  uint16_t* slab = reinterpret_cast<uint16_t*>(a.arena + it.slab_off);
  uint16_t* kbase = slab + ((int64_t)(a.layer * 2 + 0) * a.n_kv_heads + j) * region;
  uint16_t* vbase = slab + ((int64_t)(a.layer * 2 + 1) * a.n_kv_heads + j) * region;
  const bool appends = it.k_end == pos + 1;
  const int kend = appends ? pos : it.k_end;  // keys read from the slab: [k_begin, kend)
  const int b_first = it.k_begin >> 5, b_end = (kend + 31) >> 5;
  const float scale = 1.0f / sqrtf((float)DH);
  const KVStream<DH> kv{kbase, vbase, lane};

  // Everything the wave reads before its stream depends on the item only, so it is requested up
  // front (one memory latency before the first scores): the first block's keys, q, the new token's
  // k and v (every item of the row reads them; only the appending one uses them), the RoPE pairs and
  // the row's split map for the merge; the first block's values follow as soon as q is in registers.
  // Block b_first is inside the slab even when the item reads no slab key (b_first = pos / 32).
  u32x4_t K0[2 * NU], V0[NT];
  kv.load_k(K0, b_first);
  const float* qkv_row = a.qkv + (int64_t)it.row * a.ld_qkv;
  float qv[NU][8], kvals[NU][8];
  Online<DH> st;  // the new token's v lands in the accumulator: O starts as 1 x v
  {
    const float* q = qkv_row + (int64_t)(j * G + (c16 < G ? c16 : 0)) * DH;
    const float* kx = qkv_row + (int64_t)a.n_heads * DH + (int64_t)j * DH;
    const float* vx = kx + (int64_t)a.n_kv_heads * DH;
#pragma unroll
    for (int u = 0; u < NU; ++u) load8(q + 32 * u + 8 * g, qv[u]);
#pragma unroll
    for (int u = 0; u < NU; ++u) load8(kx + 32 * u + 8 * g, kvals[u]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float4 x = *reinterpret_cast<const float4*>(vx + 16 * t + 4 * g);
      st.o[t] = f32x4_t{x.x, x.y, x.z, x.w};
    }
  }
  const int2 rp = a.row_parts[it.row];

  const float2* cs = a.rope_cs + (int64_t)pos * (DH / 2);
  // lane's dims in the score product: d(u, e) = 32u + 8g + e; rotate pairs (u, u ^ PAIR) in place
  auto rotate = [&](float (&x)[NU][8]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (u & PAIR) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 c = cs[32 * u + 8 * g + e];
        const float x1 = x[u][e], x2 = x[u ^ PAIR][e];
        x[u][e] = x1 * c.x - x2 * c.y;
        x[u ^ PAIR][e] = x2 * c.x + x1 * c.y;
      }
    }
  };

  // Q^T operand: column c16 = query head j*G + c16 (zero beyond G)
  bf16x8_t qh[NU], ql[NU];
  rotate(qv);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (c16 >= G)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[u][e] = 0.f;
    split8(qv[u], qh[u], ql[u]);
  }
  kv.load_v(V0, b_first);  // (after q: its registers are free by now)

  if (!appends) {
    st.clear();
  } else {
    // The new token goes first (the softmax sum does not depend on the order): k rotated to pos and
    // rounded to bf16 on the lane's score dims, v rounded on its output dims; then stored at pos.
    rotate(kvals);
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const u32x4_t qhu = __builtin_bit_cast(u32x4_t, qh[u]), qlu = __builtin_bit_cast(u32x4_t, ql[u]);
      uint32_t kb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t b0 = f32_to_bf16(kvals[u][2 * i]), b1 = f32_to_bf16(kvals[u][2 * i + 1]);
        kb[i] = b0 | (b1 << 16);
        const float q0 = bf16_to_f32(qhu[i] & 0xFFFFu) + bf16_to_f32(qlu[i] & 0xFFFFu);
        const float q1 = bf16_to_f32(qhu[i] >> 16) + bf16_to_f32(qlu[i] >> 16);
        dot += q0 * bf16_to_f32(b0) + q1 * bf16_to_f32(b1);
      }
      if (c16 == 0)  // lanes 0, 16, 32, 48 hold every dim once
        *reinterpret_cast<uint4*>(kbase + kslab_off(pos, 32 * u + 8 * g, DH)) = uint4{kb[0], kb[1], kb[2], kb[3]};
    }
    dot += __shfl_xor(dot, 16, 64);
    dot += __shfl_xor(dot, 32, 64);
    st.m = dot * scale;  // p = exp(s - m) = 1
    st.l = 1.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t vb = f32_to_bf16(st.o[t][e]);
        st.o[t][e] = bf16_to_f32(vb);
        if (c16 == 0) vbase[vslab_off(pos, 16 * t + 4 * g + e, DH)] = (uint16_t)vb;
      }
  }

  if constexpr (PD == 1) {
    stream_blocks<DH>(kv, K0, V0, b_first, b_end, g, kend, scale, qh, ql, st);
  } else {
    u32x4_t K1[2 * NU], V1[NT];
    const int b1 = min(b_first + 1, max(b_end - 1, b_first));
    kv.load_k(K1, b1);
    kv.load_v(V1, b1);
    stream_pairs<DH>(kv, K0, V0, K1, V1, b_first, b_end, g, kend, scale, qh, ql, st);
  }
  decode_finish<DH, G>(a, it, j, rp, lane, st);
}

// ============================================================================ decode, affine 8-bit slabs
// Keys and values are stored as codes c with a (scale s, bias b) pair per key and group of 64 dims
// (value = s c + b). Codes 0..255 are exact in bf16, so the products run on the codes themselves and
// the pairs are applied around them:
//   score(key, col) = sum_g [ s_g(key) (C_g(key) . q_g(col)) + b_g(key) sum(q_g(col)) ]
//   O(d, col)       = sum_key (p s_g(d))(key) c(key, d) + sum_key p(key) b_g(d)(key)
// with C_g . q_g the product over the group's dims (one accumulator per group) and p s_g a bf16
// pair per group in place of p; the bias sums are per lane (its 8 keys) until the end. A lane's 8
// keys are those of its score rows, and the records are stored in that order, so every lane reads
// the 8 records of its lane group with plain 16-byte loads.

namespace {

// Codes of one block in registers; records of a block are staged through the wave's LDS slot (each
// lane loads 16 bytes of the block's K and V records and writes them there), and each lane reads the
// records of its lane group's 8 keys from LDS right before they are used. This keeps two blocks in
// flight within two waves per SIMD.
template <int DH, int BITS>
struct Q8Codes {
  static constexpr int NW = DH * BITS / 256;  // 16-byte code words per lane (16 / BITS fragments each)
  u32x4_t c[NW];
};

template <int DH>
struct Q8Recs {
  static constexpr int NG = DH / kQGroup;  // groups per head vector
  static constexpr int NR = 4 * NG;        // 16-byte records per lane group: 8 keys x NG pairs
  static constexpr int U = 16 * NG;        // 16-byte record units per block, K or V
  f32x4_t r[NR];
  // scale and bias of group gi for V-order key 8 * (lane / 16) + i
  CBD_DEVICE float s(int i, int gi) const { return NG == 2 ? r[i][2 * gi] : r[i >> 1][2 * (i & 1)]; }
  CBD_DEVICE float b(int i, int gi) const { return NG == 2 ? r[i][2 * gi + 1] : r[i >> 1][2 * (i & 1) + 1]; }
  // slot: 64 units, K records first (U units), then V records (U units)
  CBD_DEVICE void read(const f32x4_t* slot, int kv, int g) {
#pragma unroll
    for (int i = 0; i < NR; ++i) r[i] = slot[kv * U + NR * g + i];
  }
};

template <int DH, int BITS>
struct Q8Stream {
  const uint8_t* kbase;
  const uint8_t* vbase;
  const uint8_t* rbase;  // this lane's 16 record bytes of block 0
  int lane;
  CBD_DEVICE Q8Stream(const uint8_t* k, const uint8_t* v, int l) : kbase(k), vbase(v), lane(l) {
    constexpr int U = Q8Recs<DH>::U;
    rbase = (l < U ? k + 16 * l : v + 16 * (l < 2 * U ? l - U : 0)) + 32 * DH * BITS / 8;
  }
  CBD_DEVICE void load(Q8Codes<DH, BITS>& x, const uint8_t* base, int b) const {
    const uint8_t* p = base + (int64_t)b * q_block_bytes(DH, BITS) + 16 * lane;
#pragma unroll
    for (int i = 0; i < Q8Codes<DH, BITS>::NW; ++i) x.c[i] = load_stream(p + 1024 * i);
  }
  CBD_DEVICE void load_k(Q8Codes<DH, BITS>& x, int b) const { load(x, kbase, b); }
  CBD_DEVICE void load_v(Q8Codes<DH, BITS>& x, int b) const { load(x, vbase, b); }
  CBD_DEVICE void load_r(u32x4_t& r, int b) const { r = load_stream(rbase + (int64_t)b * q_block_bytes(DH, BITS)); }
};

// fragment `half` (0: bytes 0..7, 1: bytes 8..15) of a code word as 8 bf16 operands (exact)
CBD_DEVICE bf16x8_t code_frag(const u32x4_t& w, int half) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t x = w[2 * half + i];
    r[2 * i] = pack_bf16x2((float)(x & 255u), (float)((x >> 8) & 255u));
    r[2 * i + 1] = pack_bf16x2((float)((x >> 16) & 255u), (float)(x >> 24));
  }
  return as_frag(r);
}

// fragment q (0..3) of a 4-bit code word as 8 bf16 operands 128 + code: bf16 holds 128 + n (n < 128)
// with exponent 7 and mantissa n, so the pattern is 0x4300 | n (exact). Elements 0..3 are the low
// nibbles of the fragment's 4 bytes and 4..7 the high ones: two masks, then one byte permute (with
// 0x43 bytes from a constant) per pair of elements.
CBD_DEVICE bf16x8_t code_frag4(const u32x4_t& w, int q) {
  const uint32_t x = w[q];
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
  u32x4_t r;
  r[0] = __builtin_amdgcn_perm(0x43434343u, lo, 0x04010400u);  // bytes lo.0, 0x43, lo.1, 0x43
  r[1] = __builtin_amdgcn_perm(0x43434343u, lo, 0x04030402u);  // lo.2, 0x43, lo.3, 0x43
  r[2] = __builtin_amdgcn_perm(0x43434343u, hi, 0x04010400u);
  r[3] = __builtin_amdgcn_perm(0x43434343u, hi, 0x04030402u);
  return as_frag(r);
}

// Fragment f of a block's codes; values are code + OFF (OFF = 128 for 4-bit codes, 0 for 8-bit)
template <int DH, int BITS>
CBD_DEVICE bf16x8_t qfrag(const Q8Codes<DH, BITS>& c, int f) {
  if constexpr (BITS == 8) return code_frag(c.c[f >> 1], f & 1);
  else return code_frag4(c.c[f >> 2], f & 3);
}
template <int BITS>
constexpr float kQOff = BITS == 4 ? 128.f : 0.f;

// Raw scores of a block for the lane's 8 keys in V order (i < 4: key 4g + i, else 16 + 4g + i - 4).
template <int DH, int BITS>
CBD_DEVICE void q8_scores(const Q8Codes<DH, BITS>& K, const f32x4_t* slot, int g, const bf16x8_t (&qh)[DH / 32],
                          const bf16x8_t (&ql)[DH / 32], const float (&qs)[DH / kQGroup], float (&sv)[8]) {
  constexpr int NU = DH / 32, NG = DH / kQGroup;
  f32x4_t acc[2][NG];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) acc[h][gi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int f = h * NU + u, gi = u / 2;
      const bf16x8_t kf = qfrag<DH, BITS>(K, f);
      acc[h][gi] = mfma(kf, qh[u], acc[h][gi]);
      acc[h][gi] = mfma(kf, ql[u], acc[h][gi]);
    }
  Q8Recs<DH> R;
  R.read(slot, 0, g);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * h + e;
      float x = 0.f;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
        x += R.s(i, gi) * acc[h][gi][e] + (R.b(i, gi) - kQOff<BITS> * R.s(i, gi)) * qs[gi];
      sv[i] = x;
    }
}

// Online softmax over NB consecutive blocks from b (keys at or past lim masked): p for their keys,
// and the running state, O and the bias sums rescaled.
template <int DH, int NB>
CBD_DEVICE void q8_softmax(float (&sv)[NB][8], float (&p)[NB][8], int b, int g, int lim, float scale,
                           Online<DH>& st, float (&bacc)[DH / kQGroup]) {
  float bm = -INFINITY;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int k0 = 32 * (b + k) + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[k][e] = k0 + e < lim ? sv[k][e] * scale : -INFINITY;
      sv[k][4 + e] = k0 + 16 + e < lim ? sv[k][4 + e] * scale : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) bm = fmaxf(bm, sv[k][i]);
  }
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  const float m_new = fmaxf(st.m, bm);
  const float alpha = exp_or_zero(st.m, m_new);
  float ps = 0.f;
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[k][i] = exp_or_zero(sv[k][i], m_new);
      ps += p[k][i];
    }
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  st.l = st.l * alpha + ps;
  st.m = m_new;
#pragma unroll
  for (int t = 0; t < DH / 16; ++t) st.o[t] = st.o[t] * alpha;
#pragma unroll
  for (int gi = 0; gi < DH / kQGroup; ++gi) bacc[gi] *= alpha;
}

// O^T += codes^T (p s_g)^T per group of dims, and the bias sums, for one block.
template <int DH, int BITS>
CBD_DEVICE void q8_block_pv(const Q8Codes<DH, BITS>& V, const f32x4_t* slot, int g, const float (&p)[8], Online<DH>& st,
                            float (&bacc)[DH / kQGroup]) {
  constexpr int NG = DH / kQGroup, NT = DH / 16;
  Q8Recs<DH> R;
  R.read(slot, 1, g);
  bf16x8_t ph[NG], pl[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float pg[8], bs = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pg[i] = p[i] * R.s(i, gi);
      bs += p[i] * (R.b(i, gi) - kQOff<BITS> * R.s(i, gi));
    }
    bacc[gi] += bs;
    split8(pg, ph[gi], pl[gi]);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int gi = t / 4;
    const bf16x8_t vf = qfrag<DH, BITS>(V, t);
    st.o[t] = mfma(vf, ph[gi], st.o[t]);
    st.o[t] = mfma(vf, pl[gi], st.o[t]);
  }
}

}  // namespace

template <int DH, int G, int BITS>
__global__ __launch_bounds__(64 * kAttnWgWaves, 2) void decode_attention_q8_kernel(AttnArgs a, int n_waves) {
  constexpr int NU = DH / 32;
  constexpr int NT = DH / 16;
  constexpr int NG = DH / kQGroup;
  constexpr int PAIR = DH / 64;
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kAttnWgWaves + (threadIdx.x >> 6));
  if (w >= n_waves) return;
  const int j = w % a.n_kv_heads;
  const AttnItem it = uniform_item(a.items, w / a.n_kv_heads);
  const int pos = it.pos;
  const int64_t region = (int64_t)(it.stride / 32) * q_block_bytes(DH, BITS);
  uint8_t* slab = a.arena + it.slab_off;
  uint8_t* kbase = slab + ((int64_t)(a.layer * 2 + 0) * a.n_kv_heads + j) * region;
  uint8_t* vbase = slab + ((int64_t)(a.layer * 2 + 1) * a.n_kv_heads + j) * region;
  const bool appends = it.k_end == pos + 1;
  const int kend = appends ? pos : it.k_end;
  const int b_first = it.k_begin >> 5, b_end = (kend + 31) >> 5;
  const float scale = 1.0f / sqrtf((float)DH);
  const Q8Stream<DH, BITS> kv(kbase, vbase, lane);
  __shared__ f32x4_t q8_lds[kAttnWgWaves][2][64];
  f32x4_t* slot0 = q8_lds[threadIdx.x >> 6][0];
  f32x4_t* slot1 = q8_lds[threadIdx.x >> 6][1];

  // blocks b_first and b1 in flight from the start (records first: they are staged first)
  const int last = max(b_end - 1, b_first);
  const int b1 = min(b_first + 1, last);
  Q8Codes<DH, BITS> K0, V0, K1, V1;
  u32x4_t R0, R1;
  kv.load_r(R0, b_first);
  kv.load_r(R1, b1);
  kv.load_k(K0, b_first);
  kv.load_k(K1, b1);
  const float* qkv_row = a.qkv + (int64_t)it.row * a.ld_qkv;
  float qv[NU][8], kvals[NU][8];
  Online<DH> st;
  {
    const float* q = qkv_row + (int64_t)(j * G + (c16 < G ? c16 : 0)) * DH;
    const float* kx = qkv_row + (int64_t)a.n_heads * DH + (int64_t)j * DH;
    const float* vx = kx + (int64_t)a.n_kv_heads * DH;
#pragma unroll
    for (int u = 0; u < NU; ++u) load8(q + 32 * u + 8 * g, qv[u]);
#pragma unroll
    for (int u = 0; u < NU; ++u) load8(kx + 32 * u + 8 * g, kvals[u]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float4 x = *reinterpret_cast<const float4*>(vx + 16 * t + 4 * g);
      st.o[t] = f32x4_t{x.x, x.y, x.z, x.w};
    }
  }
  const int2 rp = a.row_parts[it.row];
  const float2* cs = a.rope_cs + (int64_t)pos * (DH / 2);
  auto rotate = [&](float (&x)[NU][8]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (u & PAIR) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 c = cs[32 * u + 8 * g + e];
        const float x1 = x[u][e], x2 = x[u ^ PAIR][e];
        x[u][e] = x1 * c.x - x2 * c.y;
        x[u ^ PAIR][e] = x2 * c.x + x1 * c.y;
      }
    }
  };

  bf16x8_t qh[NU], ql[NU];
  float qs[NG];
  rotate(qv);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) qs[gi] = 0.f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (c16 >= G)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[u][e] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[u / 2] += qv[u][e];
    split8(qv[u], qh[u], ql[u]);
  }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    qs[gi] += __shfl_xor(qs[gi], 16, 64);
    qs[gi] += __shfl_xor(qs[gi], 32, 64);
  }
  kv.load_v(V0, b_first);
  kv.load_v(V1, b1);

  float bacc[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) bacc[gi] = 0.f;
  if (!appends) {
    st.clear();
  } else {
    // the new token: k rotated and rounded to bf16, quantized per group (the 16 dims of each lane
    // group, reduced over the four lane groups), attended first with its dequantized value, stored
    rotate(kvals);
    float klo[NG], khi[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      klo[gi] = INFINITY;
      khi[gi] = -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kvals[u][e] = bf16_to_f32(f32_to_bf16(kvals[u][e]));
        klo[u / 2] = fminf(klo[u / 2], kvals[u][e]);
        khi[u / 2] = fmaxf(khi[u / 2], kvals[u][e]);
      }
    float ks[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      klo[gi] = fminf(klo[gi], __shfl_xor(klo[gi], 16, 64));
      klo[gi] = fminf(klo[gi], __shfl_xor(klo[gi], 32, 64));
      khi[gi] = fmaxf(khi[gi], __shfl_xor(khi[gi], 16, 64));
      khi[gi] = fmaxf(khi[gi], __shfl_xor(khi[gi], 32, 64));
      ks[gi] = q8_scale<BITS>(klo[gi], khi[gi]);
    }
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int gi = u / 2;
      const u32x4_t qhu = __builtin_bit_cast(u32x4_t, qh[u]), qlu = __builtin_bit_cast(u32x4_t, ql[u]);
      uint32_t cw[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t code = q8_code<BITS>(kvals[u][e], klo[gi], ks[gi]);
        if constexpr (BITS == 8) cw[e >> 2] |= code << (8 * (e & 3));
        else cw[0] |= code << (8 * (e & 3) + 4 * (e >> 2));
        const uint32_t qb = e & 1 ? qhu[e >> 1] >> 16 : qhu[e >> 1] & 0xFFFFu;
        const uint32_t lb = e & 1 ? qlu[e >> 1] >> 16 : qlu[e >> 1] & 0xFFFFu;
        dot += (bf16_to_f32(qb) + bf16_to_f32(lb)) * fmaf(ks[gi], (float)code, klo[gi]);
      }
      if (c16 == 0) {
        if constexpr (BITS == 8) *reinterpret_cast<uint2*>(kbase + kq_off(pos, 32 * u + 8 * g, DH)) = uint2{cw[0], cw[1]};
        else *reinterpret_cast<uint32_t*>(kbase + kq4_off(pos, 32 * u + 8 * g, DH)) = cw[0];
      }
    }
    dot += __shfl_xor(dot, 16, 64);
    dot += __shfl_xor(dot, 32, 64);
    st.m = dot * scale;
    st.l = 1.f;
    // v: the lane's dims 16t + 4g + e, group t / 4
    float vlo[NG], vhi[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      vlo[gi] = INFINITY;
      vhi[gi] = -INFINITY;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st.o[t][e] = bf16_to_f32(f32_to_bf16(st.o[t][e]));
        vlo[t / 4] = fminf(vlo[t / 4], st.o[t][e]);
        vhi[t / 4] = fmaxf(vhi[t / 4], st.o[t][e]);
      }
    float vs[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      vlo[gi] = fminf(vlo[gi], __shfl_xor(vlo[gi], 16, 64));
      vlo[gi] = fminf(vlo[gi], __shfl_xor(vlo[gi], 32, 64));
      vhi[gi] = fmaxf(vhi[gi], __shfl_xor(vhi[gi], 16, 64));
      vhi[gi] = fmaxf(vhi[gi], __shfl_xor(vhi[gi], 32, 64));
      vs[gi] = q8_scale<BITS>(vlo[gi], vhi[gi]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = t / 4;
        const uint32_t code = q8_code<BITS>(st.o[t][e], vlo[gi], vs[gi]);
        st.o[t][e] = fmaf(vs[gi], (float)code, vlo[gi]);
        if (c16 == 0) {
          if constexpr (BITS == 8) vbase[vq_off(pos, 16 * t + 4 * g + e, DH)] = (uint8_t)code;
          else store_nibble(vbase + vq4_off(pos, 16 * t + 4 * g + e, DH), (vslab_kk(pos) >> 2) & 1, code);
        }
      }
    if (lane == 0)
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        *reinterpret_cast<float2*>(kbase + sbq_off(pos, gi, DH, BITS)) = float2{ks[gi], klo[gi]};
        *reinterpret_cast<float2*>(vbase + sbq_off(pos, gi, DH, BITS)) = float2{vs[gi], vlo[gi]};
      }
  }

  // blocks [b_first, b_end) two at a time, the next two loading while these are used (indices past
  // the last clamp to it, so every load stays unconditional)
  int b = b_first;
  for (; b + 2 < b_end; b += 2) {
    slot0[lane] = __builtin_bit_cast(f32x4_t, R0);
    slot1[lane] = __builtin_bit_cast(f32x4_t, R1);
    __builtin_amdgcn_sched_barrier(0);
    kv.load_r(R0, b + 2);
    kv.load_r(R1, min(b + 3, last));
    __builtin_amdgcn_sched_barrier(0);
    float sv[2][8], p[2][8];
    q8_scores<DH, BITS>(K0, slot0, g, qh, ql, qs, sv[0]);
    q8_scores<DH, BITS>(K1, slot1, g, qh, ql, qs, sv[1]);
    __builtin_amdgcn_sched_barrier(0);
    kv.load_k(K0, b + 2);
    kv.load_k(K1, min(b + 3, last));
    __builtin_amdgcn_sched_barrier(0);
    q8_softmax<DH, 2>(sv, p, b, g, kend, scale, st, bacc);
    q8_block_pv<DH, BITS>(V0, slot0, g, p[0], st, bacc);
    q8_block_pv<DH, BITS>(V1, slot1, g, p[1], st, bacc);
    __builtin_amdgcn_sched_barrier(0);
    kv.load_v(V0, b + 2);
    kv.load_v(V1, min(b + 3, last));
    __builtin_amdgcn_sched_barrier(0);
  }
  slot0[lane] = __builtin_bit_cast(f32x4_t, R0);
  slot1[lane] = __builtin_bit_cast(f32x4_t, R1);
  if (b + 1 < b_end) {  // a last pair
    float sv[2][8], p[2][8];
    q8_scores<DH, BITS>(K0, slot0, g, qh, ql, qs, sv[0]);
    q8_scores<DH, BITS>(K1, slot1, g, qh, ql, qs, sv[1]);
    q8_softmax<DH, 2>(sv, p, b, g, kend, scale, st, bacc);
    q8_block_pv<DH, BITS>(V0, slot0, g, p[0], st, bacc);
    q8_block_pv<DH, BITS>(V1, slot1, g, p[1], st, bacc);
  } else if (b < b_end) {  // a last single block
    float sv[1][8], p[1][8];
    q8_scores<DH, BITS>(K0, slot0, g, qh, ql, qs, sv[0]);
    q8_softmax<DH, 1>(sv, p, b, g, kend, scale, st, bacc);
    q8_block_pv<DH, BITS>(V0, slot0, g, p[0], st, bacc);
  }
  // bias sums over the column's keys (all four lane groups), added to every dim of their group
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    bacc[gi] += __shfl_xor(bacc[gi], 16, 64);
    bacc[gi] += __shfl_xor(bacc[gi], 32, 64);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) st.o[t][e] += bacc[t / 4];
  decode_finish<DH, G>(a, it, j, rp, lane, st);
}

// ============================================================================ prefill

template <int DH>
__global__ __launch_bounds__(256, 2) void prefill_attention_kernel(AttnArgs a, int n_waves) {
  constexpr int NU = DH / 32;
  constexpr int NT = DH / 16;
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (w >= n_waves) return;
  // A tile of up to 16 queries p = pos .. k_end - 1 of one segment (global rows row, row + 1, ...);
  // the waves of a workgroup take consecutive query heads of the same tile, so the G heads of a
  // KV head read its blocks together.
  const AttnItem it = uniform_item(a.items, w / a.n_heads);
  const int h = w % a.n_heads, j = h / (a.n_heads / a.n_kv_heads);
  const int n_q = it.k_end - it.pos;
  const int64_t region = (int64_t)it.stride * DH;
  const uint16_t* slab = reinterpret_cast<const uint16_t*>(a.arena + it.slab_off);
  const KVStream<DH> kv{slab + ((int64_t)(a.layer * 2 + 0) * a.n_kv_heads + j) * region,
                        slab + ((int64_t)(a.layer * 2 + 1) * a.n_kv_heads + j) * region, lane};
  // a forked sequence: blocks [0, pb) from the parent's slab, the rest from its own
  const int pb = it.pre_end >> 5;
  const int64_t pregion = (int64_t)it.pre_stride * DH;
  const uint16_t* pslab = reinterpret_cast<const uint16_t*>(a.arena + it.pre_off);
  const KVStream<DH> kp{pslab + ((int64_t)(a.layer * 2 + 0) * a.n_kv_heads + j) * pregion,
                        pslab + ((int64_t)(a.layer * 2 + 1) * a.n_kv_heads + j) * pregion, lane};
  u32x4_t K0[2 * NU], V0[NT];
  if (pb > 0) kp.load_k(K0, 0);
  else kv.load_k(K0, 0);
  // Q^T operand: column c16 = query pos + c16 (zero past the tile), already rotated
  bf16x8_t qh[NU], ql[NU];
  {
    const float* q = a.qkv + (int64_t)(it.row + min(c16, n_q - 1)) * a.ld_qkv + (int64_t)h * DH;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float qv[8];
      load8(q + 32 * u + 8 * g, qv);
      if (c16 >= n_q)
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = 0.f;
      split8(qv, qh[u], ql[u]);
    }
  }
  if (pb > 0) kp.load_v(V0, 0);
  else kv.load_v(V0, 0);
  Online<DH> st;
  st.clear();
  // causal: column c16 sees keys 0 .. pos + c16 of its own segment (columns past the tile see none)
  const int lim = c16 < n_q ? it.pos + c16 + 1 : 0;
  const float scale = 1.0f / sqrtf((float)DH);
  if (pb > 0) {
    stream_blocks<DH>(kp, K0, V0, 0, pb, g, lim, scale, qh, ql, st);
    kv.load_k(K0, pb);
    kv.load_v(V0, pb);
  }
  stream_blocks<DH>(kv, K0, V0, pb, (it.k_end + 31) >> 5, g, lim, scale, qh, ql, st);
  if (c16 < n_q) store_out<DH>(a, it.row + c16, h, g, st.o, 1.0f / st.l);
}

// Prefill over affine 8-bit slabs: the tile and column layout of prefill_attention_kernel, blocks
// streamed one at a time through the code products of the decode kernel.
template <int DH, int BITS>
__global__ __launch_bounds__(256, 2) void prefill_attention_q8_kernel(AttnArgs a, int n_waves) {
  constexpr int NU = DH / 32;
  constexpr int NT = DH / 16;
  constexpr int NG = DH / kQGroup;
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  __shared__ f32x4_t q8_lds[4][64];
  f32x4_t* slot = q8_lds[threadIdx.x >> 6];
  if (w >= n_waves) return;
  const AttnItem it = uniform_item(a.items, w / a.n_heads);
  const int h = w % a.n_heads, j = h / (a.n_heads / a.n_kv_heads);
  const int n_q = it.k_end - it.pos;
  const int64_t region = (int64_t)(it.stride / 32) * q_block_bytes(DH, BITS);
  const uint8_t* slab = a.arena + it.slab_off;
  const Q8Stream<DH, BITS> kv(slab + ((int64_t)(a.layer * 2 + 0) * a.n_kv_heads + j) * region,
                        slab + ((int64_t)(a.layer * 2 + 1) * a.n_kv_heads + j) * region, lane);
  // a forked sequence: blocks [0, pb) from the parent's slab, the rest from its own
  const int pb = it.pre_end >> 5;
  const int64_t pregion = (int64_t)(it.pre_stride / 32) * q_block_bytes(DH, BITS);
  const uint8_t* pslab = a.arena + it.pre_off;
  const Q8Stream<DH, BITS> kp(pslab + ((int64_t)(a.layer * 2 + 0) * a.n_kv_heads + j) * pregion,
                        pslab + ((int64_t)(a.layer * 2 + 1) * a.n_kv_heads + j) * pregion, lane);
  Q8Codes<DH, BITS> K0, V0;
  u32x4_t R0;
  (pb > 0 ? kp : kv).load_r(R0, 0);
  (pb > 0 ? kp : kv).load_k(K0, 0);
  bf16x8_t qh[NU], ql[NU];
  float qs[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) qs[gi] = 0.f;
  {
    const float* q = a.qkv + (int64_t)(it.row + min(c16, n_q - 1)) * a.ld_qkv + (int64_t)h * DH;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float qv[8];
      load8(q + 32 * u + 8 * g, qv);
      if (c16 >= n_q)
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) qs[u / 2] += qv[e];
      split8(qv, qh[u], ql[u]);
    }
  }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    qs[gi] += __shfl_xor(qs[gi], 16, 64);
    qs[gi] += __shfl_xor(qs[gi], 32, 64);
  }
  (pb > 0 ? kp : kv).load_v(V0, 0);
  Online<DH> st;
  st.clear();
  float bacc[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) bacc[gi] = 0.f;
  const int lim = c16 < n_q ? it.pos + c16 + 1 : 0;
  const int b_end = (it.k_end + 31) >> 5;
  for (int b = 0; b < b_end; ++b) {
    const int nb = min(b + 1, b_end - 1);
    const Q8Stream<DH, BITS>& nx = nb < pb ? kp : kv;  // the slab that holds the next block
    slot[lane] = __builtin_bit_cast(f32x4_t, R0);
    nx.load_r(R0, nb);
    float sv[1][8], p[1][8];
    q8_scores<DH, BITS>(K0, slot, g, qh, ql, qs, sv[0]);
    nx.load_k(K0, nb);
    q8_softmax<DH, 1>(sv, p, b, g, lim, 1.0f / sqrtf((float)DH), st, bacc);
    q8_block_pv<DH, BITS>(V0, slot, g, p[0], st, bacc);
    nx.load_v(V0, nb);
  }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    bacc[gi] += __shfl_xor(bacc[gi], 16, 64);
    bacc[gi] += __shfl_xor(bacc[gi], 32, 64);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) st.o[t][e] += bacc[t / 4];
  if (c16 < n_q) store_out<DH>(a, it.row + c16, h, g, st.o, 1.0f / st.l);
}

template <int DH>
static hipError_t launch_decode_dh(int G, dim3 grid, int n_waves, hipStream_t st, const AttnArgs& a) {
  switch (G) {
    case 1: launch_kernel((decode_attention_kernel<DH, 1, CBD_ATTN_PD>), grid, dim3(64 * kAttnWgWaves), 0, st, a, n_waves); break;
    case 2: launch_kernel((decode_attention_kernel<DH, 2, CBD_ATTN_PD>), grid, dim3(64 * kAttnWgWaves), 0, st, a, n_waves); break;
    case 4: launch_kernel((decode_attention_kernel<DH, 4, CBD_ATTN_PD>), grid, dim3(64 * kAttnWgWaves), 0, st, a, n_waves); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_attention(const AttnArgs& a, int n_items, int head_dim, hipStream_t st) {
  const int G = a.n_heads / a.n_kv_heads;
  const int n_waves = n_items * a.n_kv_heads;
  const dim3 grid((n_waves + kAttnWgWaves - 1) / kAttnWgWaves);
  if (head_dim == 128) return launch_decode_dh<128>(G, grid, n_waves, st, a);
  if (head_dim == 64) return launch_decode_dh<64>(G, grid, n_waves, st, a);
  return hipErrorInvalidValue;
}

template <int DH, int BITS>
static hipError_t launch_decode_q8_dh(int G, dim3 grid, int n_waves, hipStream_t st, const AttnArgs& a) {
  switch (G) {
    case 1: launch_kernel((decode_attention_q8_kernel<DH, 1, BITS>), grid, dim3(64 * kAttnWgWaves), 0, st, a, n_waves); break;
    case 2: launch_kernel((decode_attention_q8_kernel<DH, 2, BITS>), grid, dim3(64 * kAttnWgWaves), 0, st, a, n_waves); break;
    case 4: launch_kernel((decode_attention_q8_kernel<DH, 4, BITS>), grid, dim3(64 * kAttnWgWaves), 0, st, a, n_waves); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_attention_q8(const AttnArgs& a, int n_items, int head_dim, int bits, hipStream_t st) {
  const int G = a.n_heads / a.n_kv_heads;
  const int n_waves = n_items * a.n_kv_heads;
  const dim3 grid((n_waves + kAttnWgWaves - 1) / kAttnWgWaves);
  if (bits == 8 && head_dim == 128) return launch_decode_q8_dh<128, 8>(G, grid, n_waves, st, a);
  if (bits == 8 && head_dim == 64) return launch_decode_q8_dh<64, 8>(G, grid, n_waves, st, a);
  if (bits == 4 && head_dim == 128) return launch_decode_q8_dh<128, 4>(G, grid, n_waves, st, a);
  if (bits == 4 && head_dim == 64) return launch_decode_q8_dh<64, 4>(G, grid, n_waves, st, a);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_attention_q8(const AttnArgs& a, int n_items, int head_dim, int bits, hipStream_t st) {
  const int n_waves = n_items * a.n_heads;
  const dim3 grid((n_waves + 3) / 4);
  if (bits == 8 && head_dim == 128) launch_kernel((prefill_attention_q8_kernel<128, 8>), grid, dim3(256), 0, st, a, n_waves);
  else if (bits == 8 && head_dim == 64) launch_kernel((prefill_attention_q8_kernel<64, 8>), grid, dim3(256), 0, st, a, n_waves);
  else if (bits == 4 && head_dim == 128) launch_kernel((prefill_attention_q8_kernel<128, 4>), grid, dim3(256), 0, st, a, n_waves);
  else if (bits == 4 && head_dim == 64) launch_kernel((prefill_attention_q8_kernel<64, 4>), grid, dim3(256), 0, st, a, n_waves);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefill_attention(const AttnArgs& a, int n_items, int head_dim, hipStream_t st) {
  const int n_waves = n_items * a.n_heads;
  const dim3 grid((n_waves + 3) / 4);
  if (head_dim == 128) launch_kernel((prefill_attention_kernel<128>), grid, dim3(256), 0, st, a, n_waves);
  else if (head_dim == 64) launch_kernel((prefill_attention_kernel<64>), grid, dim3(256), 0, st, a, n_waves);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cbd
