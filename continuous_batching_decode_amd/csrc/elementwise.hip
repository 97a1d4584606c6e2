// Row-wise kernels of the decode step: embedding gather (with the first
// norm's gain and sums of squares), RoPE at each row's own position + K/V
// append into its slab, greedy argmax, activation plane split, and slab
// scatter/gather for seeding and inspection.
//
// Position discipline (page "Batching", section 5): a row's position is read
// once per step from its metadata and used for both the query and the key
// rotation and for the slab slot the key is written to.
#include "common.h"
#include "kernels.h"

namespace cbd {

namespace {

CBD_DEVICE void split_store(uint16_t* hi, uint16_t* lo, float v) {
  const uint32_t h = f32_to_bf16(v);
  *hi = (uint16_t)h;
  *lo = (uint16_t)f32_to_bf16(v - bf16_to_f32(h));
}

}  // namespace

// One block per row. Each thread takes 8 consecutive features at a time (one 16-byte load of the
// embedding row and of the gain): it writes them to h, the 8 hi and 8 lo values of gain * h (16
// contiguous bytes each in the fragment layout), and with its neighbour lane (the other half of a
// 16-feature group) the group's sum of squares. d % 16 == 0.
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* tokens, const uint16_t* embed, int vocab, int d,
                                                    const uint16_t* gain, float* h, uint16_t* xp, int64_t plane,
                                                    float* ss, int ss_ld) {
  const int r = blockIdx.x;
  int tok = tokens[r];
  tok = tok < 0 ? 0 : (tok >= vocab ? vocab - 1 : tok);  // ids stay on the device: clamp out-of-range ids
  const uint16_t* e = embed + (int64_t)tok * d;
  float* hrow = h + (int64_t)r * d;
  // chunks of 8 features; whole waves take part in every round (the sum pairs lanes t, t ^ 1)
  const int chunks = d / 8, rounds = (chunks + 255) / 256;
  for (int k = 0; k < rounds; ++k) {
    const int t = threadIdx.x + 256 * k;
    const bool on = t < chunks;
    const int tc = on ? t : 0;
    const uint4 ev = *reinterpret_cast<const uint4*>(e + 8 * tc);
    const uint4 gv = *reinterpret_cast<const uint4*>(gain + 8 * tc);
    const uint32_t ew[4] = {ev.x, ev.y, ev.z, ev.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
    float v[8], y[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(ew[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_to_f32(ew[i] >> 16);
      y[2 * i] = v[2 * i] * bf16_to_f32(gw[i] & 0xFFFFu);
      y[2 * i + 1] = v[2 * i + 1] * bf16_to_f32(gw[i] >> 16);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i] * v[i];
    s += __shfl_xor(s, 1, 64);  // the 16-feature group: chunks 2u and 2u + 1
    if (on) {
      *reinterpret_cast<float4*>(hrow + 8 * t) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(hrow + 8 * t + 4) = make_float4(v[4], v[5], v[6], v[7]);
      uint4 hi, lo;
      hi.x = pack_bf16x2(y[0], y[1]);
      hi.y = pack_bf16x2(y[2], y[3]);
      hi.z = pack_bf16x2(y[4], y[5]);
      hi.w = pack_bf16x2(y[6], y[7]);
      lo.x = pack_bf16x2(y[0] - bf16_to_f32(hi.x & 0xFFFFu), y[1] - bf16_to_f32(hi.x >> 16));
      lo.y = pack_bf16x2(y[2] - bf16_to_f32(hi.y & 0xFFFFu), y[3] - bf16_to_f32(hi.y >> 16));
      lo.z = pack_bf16x2(y[4] - bf16_to_f32(hi.z & 0xFFFFu), y[5] - bf16_to_f32(hi.z >> 16));
      lo.w = pack_bf16x2(y[6] - bf16_to_f32(hi.w & 0xFFFFu), y[7] - bf16_to_f32(hi.w >> 16));
      const int64_t o = xfrag_off(r, 8 * t, d);  // features 8t .. 8t + 7 are contiguous there
      *reinterpret_cast<uint4*>(xp + o) = hi;
      *reinterpret_cast<uint4*>(xp + plane + o) = lo;
      if ((t & 1) == 0) ss[(int64_t)(t >> 1) * ss_ld + r] = s;
    }
  }
}

__global__ __launch_bounds__(256) void split_planes_kernel(const float* x, int K, uint16_t* out, int64_t plane) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < K; i += 256) {
    const int64_t o = xfrag_off(r, i, K);
    split_store(out + o, out + plane + o, x[(int64_t)r * K + i]);
  }
}

// Copy activation row row_idx[r] (fragment-major planes, width d) to row r of the output planes,
// with its per-16-feature sums of squares.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* x, int64_t x_plane, const float* ss,
                                                          int ss_ld, const int32_t* row_idx, int d, uint16_t* out,
                                                          int64_t out_plane, float* ss_out, int ss_out_ld) {
  const int r = blockIdx.x;
  const int src = row_idx[r];
  for (int f = threadIdx.x; f < d; f += 256) {
    const int64_t i = xfrag_off(src, f, d), o = xfrag_off(r, f, d);
    out[o] = x[i];
    out[o + out_plane] = x[i + x_plane];
  }
  for (int t = threadIdx.x; t < d / 16; t += 256) ss_out[(int64_t)t * ss_out_ld + r] = ss[(int64_t)t * ss_ld + src];
}

// rope_cs: [max_pos][head_dim/2] (cos, sin) pairs, fp32 values of angles computed in fp64.
__global__ __launch_bounds__(256) void rope_append_kernel(float* qkv, int ld_qkv, const RowMeta* meta, int n_heads,
                                                          int n_kv_heads, int head_dim, int layer, uint8_t* arena,
                                                          const float2* rope_cs) {
  const int r = blockIdx.x;
  const RowMeta m = meta[r];
  const int half = head_dim >> 1;
  const float2* cs = rope_cs + (int64_t)m.pos * half;
  float* q = qkv + (int64_t)r * ld_qkv;
  float* k = q + n_heads * head_dim;
  const float* v = k + n_kv_heads * head_dim;
  // queries: rotate in place, kept fp32
  for (int idx = threadIdx.x; idx < n_heads * half; idx += 256) {
    const int hh = idx / half, i = idx - hh * half;
    float* x = q + hh * head_dim;
    const float2 c = cs[i];
    const float x1 = x[i], x2 = x[i + half];
    x[i] = x1 * c.x - x2 * c.y;
    x[i + half] = x2 * c.x + x1 * c.y;
  }
  // keys: rotate, round to bf16, write to the slab at pos; values: round and write
  uint16_t* slab = reinterpret_cast<uint16_t*>(arena + m.slab_off);
  const int64_t region = (int64_t)m.stride * head_dim;
  uint16_t* kbase = slab + (int64_t)(layer * 2 + 0) * n_kv_heads * region;
  uint16_t* vbase = slab + (int64_t)(layer * 2 + 1) * n_kv_heads * region;
  for (int idx = threadIdx.x; idx < n_kv_heads * half; idx += 256) {
    const int j = idx / half, i = idx - j * half;
    const float* x = k + j * head_dim;
    const float2 c = cs[i];
    const float x1 = x[i], x2 = x[i + half];
    uint16_t* dst = kbase + j * region;
    dst[kslab_off(m.pos, i, head_dim)] = (uint16_t)f32_to_bf16(x1 * c.x - x2 * c.y);
    dst[kslab_off(m.pos, i + half, head_dim)] = (uint16_t)f32_to_bf16(x2 * c.x + x1 * c.y);
  }
  for (int idx = threadIdx.x; idx < n_kv_heads * head_dim; idx += 256) {
    const int j = idx / head_dim, i = idx - j * head_dim;
    vbase[j * region + vslab_off(m.pos, i, head_dim)] = (uint16_t)f32_to_bf16(v[idx]);
  }
}

// Greedy argmax, lowest index on ties. Row r is cut into P segments, one block each: strict >
// keeps the first maximum a thread sees, and across threads and blocks equal values resolve to
// the lower index. Each block publishes (max, index) with agent-scope stores; the last block of the
// row (arrival counter) reduces the P pairs in the same way and resets the counter.
namespace {
CBD_DEVICE void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}
CBD_DEVICE void block_best(float& bv, int& bi, float* sv, int* si) {
  sv[threadIdx.x] = bv;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      float mv = sv[threadIdx.x];
      int mi = si[threadIdx.x];
      better(mv, mi, sv[threadIdx.x + s], si[threadIdx.x + s]);
      sv[threadIdx.x] = mv;
      si[threadIdx.x] = mi;
    }
    __syncthreads();
  }
  bv = sv[0];
  bi = si[0];
}
}  // namespace

__global__ __launch_bounds__(256) void argmax_kernel(const float* logits, int vocab, int seg, float* part,
                                                     int32_t* counters, int32_t* out) {
  __shared__ float sv[256];
  __shared__ int si[256];
  __shared__ int s_last;
  const int r = blockIdx.y, P = gridDim.x, b = blockIdx.x;
  const float* row = logits + (int64_t)r * vocab;
  const int v0 = b * seg, v1 = min(vocab, v0 + seg);
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int v = v0 + threadIdx.x * 4; v < v1; v += 256 * 4) {
    const float4 x = *reinterpret_cast<const float4*>(row + v);
    better(best, bi, x.x, v);
    better(best, bi, x.y, v + 1);
    better(best, bi, x.z, v + 2);
    better(best, bi, x.w, v + 3);
  }
  block_best(best, bi, sv, si);
  if (threadIdx.x == 0) {
    store_agent_x2(part, (int)(((int64_t)r * P + b) * 8), float2{best, __int_as_float(bi)});
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the pair is stored before arrival counts
    s_last = __hip_atomic_fetch_add(counters + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == P - 1;
  }
  __syncthreads();
  if (!s_last) return;
  best = -INFINITY;
  bi = 0x7FFFFFFF;
  for (int q = threadIdx.x; q < P; q += 256) {
    const float2 x = load_agent_x2(part, (int)(((int64_t)r * P + q) * 8));
    better(best, bi, x.x, __float_as_int(x.y));
  }
  block_best(best, bi, sv, si);
  if (threadIdx.x == 0) {
    out[r] = bi == 0x7FFFFFFF ? 0 : bi;  // every logit NaN: token 0
    __hip_atomic_store(counters + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// canonical [L, n, Hkv, Dh] <-> slab [L][2][Hkv][cap][Dh] at positions [pos, pos+n); 16-byte moves
__global__ __launch_bounds__(256) void slab_copy_kernel(uint8_t* arena, int64_t slab_off, int stride, int pos,
                                                        int n, int n_kv_heads, int head_dim, const uint16_t* k_in,
                                                        const uint16_t* v_in, uint16_t* k_out, uint16_t* v_out) {
  const int t = blockIdx.x, l = blockIdx.y, kv = blockIdx.z;
  const int chunks = n_kv_heads * head_dim / 8;
  uint16_t* slab = reinterpret_cast<uint16_t*>(arena + slab_off);
  const int64_t region = (int64_t)stride * head_dim;
  const int64_t canon = ((int64_t)l * n + t) * n_kv_heads * head_dim;
  const int key = pos + t;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const int j = (c * 8) / head_dim, i = (c * 8) - j * head_dim;
    uint16_t* base = slab + ((int64_t)(l * 2 + kv) * n_kv_heads + j) * region;
    if (kv == 0) {  // 8 consecutive dims of a key are contiguous in a K fragment
      uint16_t* s = base + kslab_off(key, i, head_dim);
      if (k_in)
        *reinterpret_cast<uint4*>(s) = *reinterpret_cast<const uint4*>(k_in + canon + c * 8);
      else
        *reinterpret_cast<uint4*>(k_out + canon + c * 8) = *reinterpret_cast<const uint4*>(s);
    } else {  // ... but 16 bytes apart in a V fragment
      for (int e = 0; e < 8; ++e) {
        uint16_t* s = base + vslab_off(key, i + e, head_dim);
        if (v_in)
          *s = v_in[canon + c * 8 + e];
        else
          v_out[canon + c * 8 + e] = *s;
      }
    }
  }
}

hipError_t launch_embed(const int32_t* tokens, int rows, const uint16_t* embed, int vocab, int d,
                        const uint16_t* gain, float* h, uint16_t* xplanes, int64_t plane, float* ss, int ss_ld,
                        hipStream_t st) {
  launch_kernel(embed_kernel, dim3(rows), dim3(256), 0, st, tokens, embed, vocab, d, gain, h, xplanes, plane, ss,
                     ss_ld);
  return hipGetLastError();
}

hipError_t launch_split_planes(const float* x, int rows, int K, uint16_t* out, int64_t plane, hipStream_t st) {
  launch_kernel(split_planes_kernel, dim3(rows), dim3(256), 0, st, x, K, out, plane);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* x, int64_t x_plane, const float* ss, int ss_ld, const int32_t* row_idx,
                              int rows, int d, uint16_t* out, int64_t out_plane, float* ss_out, int ss_out_ld,
                              hipStream_t st) {
  launch_kernel(gather_rows_kernel, dim3(rows), dim3(256), 0, st, x, x_plane, ss, ss_ld, row_idx, d, out,
                     out_plane, ss_out, ss_out_ld);
  return hipGetLastError();
}

hipError_t launch_rope_append(float* qkv, int ld_qkv, const RowMeta* meta, int rows, int n_heads, int n_kv_heads,
                              int head_dim, int layer, uint8_t* arena, const float* rope_cs, hipStream_t st) {
  launch_kernel(rope_append_kernel, dim3(rows), dim3(256), 0, st, qkv, ld_qkv, meta, n_heads, n_kv_heads,
                     head_dim, layer, arena, reinterpret_cast<const float2*>(rope_cs));
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int rows, int vocab, float* part, int32_t* counters, int32_t* out,
                         hipStream_t st) {
  // segments of a multiple of 4 logits, 4096 or more each, at most kArgmaxSegments per row
  int P = (vocab + 4095) / 4096;
  P = P < 1 ? 1 : (P > kArgmaxSegments ? kArgmaxSegments : P);
  const int seg = ((vocab + P - 1) / P + 3) / 4 * 4;
  P = (vocab + seg - 1) / seg;
  launch_kernel(argmax_kernel, dim3(P, rows), dim3(256), 0, st, logits, vocab, seg, part, counters, out);
  return hipGetLastError();
}

hipError_t launch_slab_copy(uint8_t* arena, int64_t slab_off, int stride, int pos, int n, int n_layers,
                            int n_kv_heads, int head_dim, const uint16_t* k_in, const uint16_t* v_in, uint16_t* k_out,
                            uint16_t* v_out, hipStream_t st) {
  launch_kernel(slab_copy_kernel, dim3(n, n_layers, 2), dim3(256), 0, st, arena, slab_off, stride, pos, n,
                     n_kv_heads, head_dim, k_in, v_in, k_out, v_out);
  return hipGetLastError();
}


// ============================================================================ seeded top-p sampling
// Row r (one workgroup of 1024 threads): temperature T_r, nucleus mass p_r, draw from Philox4x64-10
// with key (seed_r, 0) and counter (index_r, 0, 0, 0). T_r = 0 is greedy (lowest id among maxima).
// Otherwise e_i = exp(z_i - max z) with z = logit / T, in fixed point w_i = floor(e_i 2^40) (integer
// masses: every comparison below is exact and order-free). The nucleus is the shortest prefix of the
// ids ordered by e descending (ties: lower id first) whose mass reaches floor(p_r W), W = sum w; the
// token is the first of that order whose running mass exceeds floor(u M), M = nucleus mass, u the
// 24-bit draw. Both searches descend the bit patterns of e (order-preserving for positive floats) in
// three radix levels of 11, 11 and 10 bits with mass and count histograms in LDS; the ties at the
// final pattern are resolved in id order with a scan of per-thread counts over contiguous chunks.
namespace {
constexpr int kSampleThreads = 1024;
constexpr uint64_t kFix = 1ull << 40;

CBD_DEVICE uint64_t mulhi64(uint64_t a, uint64_t b) { return __umul64hi(a, b); }

// Philox4x64-10 word 0 for counter (ctr, 0, 0, 0) and key (k0, 0)
CBD_DEVICE uint64_t philox_word0(uint64_t ctr, uint64_t k0) {
  uint64_t c0 = ctr, c1 = 0, c2 = 0, c3 = 0, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t h0 = mulhi64(c0, 0xD2E7470EE14C6C93ull), l0 = c0 * 0xD2E7470EE14C6C93ull;
    const uint64_t h1 = mulhi64(c2, 0xCA5A826395121157ull), l1 = c2 * 0xCA5A826395121157ull;
    const uint64_t n0 = h1 ^ c1 ^ k0, n2 = h0 ^ c3 ^ k1;
    c0 = n0;
    c1 = l1;
    c2 = n2;
    c3 = l0;
    k0 += 0x9E3779B97F4A7C15ull;
    k1 += 0xBB67AE8584CAA73Bull;
  }
  return c0;
}

template <typename T>
CBD_DEVICE T block_sum(T v, T* red) {  // fixed order: lanes by xor tree, then the 16 waves in order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  T s = 0;
  for (int i = 0; i < kSampleThreads / 64; ++i) s += red[i];
  return s;
}

CBD_DEVICE float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
  for (int i = 1; i < kSampleThreads / 64; ++i) m = fmaxf(m, red[i]);
  return m;
}
}  // namespace

__global__ __launch_bounds__(kSampleThreads) void sample_top_p_kernel(const float* logits, int vocab, SampleArgs p,
                                                                      int32_t* out) {
  __shared__ uint64_t hmass[2048];
  __shared__ uint32_t hcount[1024];
  __shared__ uint64_t red64[kSampleThreads / 64];
  __shared__ float redf[kSampleThreads / 64];
  __shared__ uint32_t red32[kSampleThreads / 64];
  __shared__ uint32_t s_bin;
  __shared__ uint64_t s_above;
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* row = logits + (int64_t)r * vocab;
  const float4* row4 = reinterpret_cast<const float4*>(row);
  const float temp = p.temperature[r];
  const int n4 = vocab >> 2;  // vocab % 4 == 0 (checked by the host)
  // Every pass visits the thread's float4s q = tid + 1024 i in increasing order, 8 loads in flight
  // (clamped indices, so the loads are unconditional).
  constexpr int UNR = 8;
  auto pass = [&](auto&& visit) {
    for (int q0 = tid; q0 < n4; q0 += UNR * kSampleThreads) {
      float4 xb[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) xb[u] = row4[min(q0 + u * kSampleThreads, n4 - 1)];
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        if (q0 + u * kSampleThreads < n4) {
          const int v = 4 * (q0 + u * kSampleThreads);
          visit(xb[u].x, v);
          visit(xb[u].y, v + 1);
          visit(xb[u].z, v + 2);
          visit(xb[u].w, v + 3);
        }
    }
  };

  if (temp == 0.f) {  // greedy: strict > in id order per thread, then (max, lowest id) over the block
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    pass([&](float x, int v) {
      if (x > best || (x == best && v < bi)) {
        best = x;
        bi = v;
      }
    });
    const float m = block_max(best, redf);
    uint32_t cand = (best == m) ? (uint32_t)bi : 0x7FFFFFFFu;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cand = min(cand, (uint32_t)__shfl_xor((int)cand, o, 64));
    __syncthreads();
    if ((tid & 63) == 0) red32[tid >> 6] = cand;
    __syncthreads();
    if (tid == 0) {
      uint32_t bb = red32[0];
      for (int i = 1; i < kSampleThreads / 64; ++i) bb = min(bb, red32[i]);
      out[r] = bb == 0x7FFFFFFFu ? 0 : (int32_t)bb;  // every logit NaN: token 0
    }
    return;
  }

  const float inv_t = 1.0f / temp;
  // max of z (NaN logits are skipped: they never win and weigh nothing)
  float mz = -INFINITY;
  pass([&](float x, int) { mz = fmaxf(mz, x * inv_t); });
  mz = block_max(mz, redf);
  // bit pattern of e = exp(z - max z) (0 for NaN) and its fixed-point mass floor(e 2^40): the
  // mantissa shifted by the exponent (exact; 0 below 2^-40)
  auto weight = [&](float x, uint32_t& bits) -> uint64_t {
    const float e = __expf(x * inv_t - mz);
    bits = (e == e) ? __float_as_uint(e) : 0u;
    const int ex = (int)(bits >> 23);  // biased exponent; e <= 1 so ex <= 127
    const uint64_t man = (uint64_t)((bits & 0x7FFFFFu) | 0x800000u);
    const int sh = ex - 110;  // e 2^40 = man 2^(ex - 127 - 23 + 40)
    return ex == 0 ? 0ull : sh >= 0 ? man << sh : (sh > -24 ? man >> (-sh) : 0ull);
  };
  uint64_t tw = 0;
  pass([&](float x, int) {
    uint32_t bb;
    tw += weight(x, bb);
  });
  const uint64_t W = block_sum<uint64_t>(tw, red64);

  // One radix descent over the patterns of positive weights: the largest pattern P such that the
  // mass of the patterns above P (the ties at `cap_bits` counted as `cap_excess` lighter) plus the
  // mass at P crosses `target` (>= when ge, else >). Returns P, the mass strictly above it and the
  // number of tokens at it.
  auto descend = [&](uint64_t target, bool ge, uint32_t cap_bits, uint64_t cap_excess, uint32_t& pat,
                     uint64_t& above, uint32_t& cnt) {
    uint32_t prefix = 0;
    above = 0;
    const int widths[3] = {11, 11, 10};
    int shift = 32;
    for (int lv = 0; lv < 3; ++lv) {
      const int wb = widths[lv];
      shift -= wb;
      const int nb = 1 << wb;
      for (int i = tid; i < nb; i += kSampleThreads) {
        hmass[i] = 0;
        if (lv == 2) hcount[i] = 0;
      }
      __syncthreads();
      pass([&](float x, int) {
        uint32_t bb;
        const uint64_t w = weight(x, bb);
        if (w != 0 && (shift + wb == 32 || (bb >> (shift + wb)) == prefix)) {
          const int bin = (bb >> shift) & (nb - 1);
          atomicAdd(reinterpret_cast<unsigned long long*>(&hmass[bin]), (unsigned long long)w);
          if (lv == 2) atomicAdd(&hcount[bin], 1u);
        }
      });
      __syncthreads();
      if (tid == 0 && cap_excess && (shift + wb == 32 || (cap_bits >> (shift + wb)) == prefix))
        hmass[(cap_bits >> shift) & (nb - 1)] -= cap_excess;
      __syncthreads();
      // running mass from the top bin down: thread t holds bins nb-1-2t and nb-2-2t; a scan over the
      // threads gives each pair the mass above it, and the one pair where the running mass crosses
      // the target names the bin
      const int bh = nb - 1 - 2 * tid, bl = bh - 1;
      const uint64_t mh = bh >= 0 ? hmass[bh] : 0ull, ml = bl >= 0 ? hmass[bl] : 0ull;
      const uint64_t pr = mh + ml;
      uint64_t incl = pr;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(incl, o, 64);
        if ((tid & 63) >= o) incl += y;
      }
      if ((tid & 63) == 63) red64[tid >> 6] = incl;
      if (tid == 0) {
        s_bin = 0;  // (unreachable fallback: the lowest bin)
        s_above = above;
      }
      __syncthreads();
      uint64_t a0 = above + incl - pr;
      for (int i = 0; i < (tid >> 6); ++i) a0 += red64[i];
      auto crossed = [&](uint64_t m) { return ge ? m >= target : m > target; };
      if (bh >= 0 && !crossed(a0)) {
        if (crossed(a0 + mh)) {
          s_bin = (uint32_t)bh;
          s_above = a0;
        } else if (bl >= 0 && crossed(a0 + pr)) {
          s_bin = (uint32_t)bl;
          s_above = a0 + mh;
        }
      }
      __syncthreads();
      prefix = (prefix << wb) | s_bin;
      above = s_above;
      if (lv == 2) cnt = hcount[s_bin];
      __syncthreads();
    }
    pat = prefix;
  };
  auto fixed_of = [&](uint32_t bits) -> uint64_t {  // the weight of a pattern (as in weight())
    const int ex = (int)(bits >> 23);
    const uint64_t man = (uint64_t)((bits & 0x7FFFFFu) | 0x800000u);
    const int sh = ex - 110;
    return ex == 0 ? 0ull : sh >= 0 ? man << sh : (sh > -24 ? man >> (-sh) : 0ull);
  };

  // nucleus boundary: pattern theta, the mass above it, its tie count and how many ties it keeps
  const uint64_t target = (uint64_t)((double)p.top_p[r] * (double)W);
  uint32_t th, nt;
  uint64_t above_th;
  descend(target > 0 ? target : 1, true, 0u, 0ull, th, above_th, nt);
  const uint64_t wth = fixed_of(th);
  uint64_t keep = wth ? (target > above_th ? (target - above_th + wth - 1) / wth : 1) : nt;
  keep = keep < 1 ? 1 : (keep > nt ? nt : keep);
  const uint64_t M = above_th + keep * wth;
  // the draw and its point t = floor(u M) in the nucleus mass (exact: u has 24 bits)
  const uint64_t u24 = philox_word0(p.index[r], p.seed[r]) >> 40;
  const uint64_t t = u24 * (M >> 24) + ((u24 * (M & 0xFFFFFFull)) >> 24);
  uint32_t ph, nph;
  uint64_t above_ph;
  descend(t, false, th, (uint64_t)(nt - keep) * wth, ph, above_ph, nph);
  const uint64_t wph = fixed_of(ph);
  uint64_t j = wph ? (t - above_ph) / wph : 0;
  const uint64_t avail = ph == th ? keep : nph;
  if (j >= avail) j = avail ? avail - 1 : 0;
  // the j-th id (ascending) among the tokens with pattern ph: per-thread counts over contiguous
  // chunks of CH float4s, an exclusive scan, then the owner picks (token 0 stands if no weight is
  // positive)
  if (tid == 0) out[r] = 0;
  const int CH = (n4 + kSampleThreads - 1) / kSampleThreads;
  const int c0 = tid * CH, c1 = min(n4, c0 + CH);
  uint32_t mine = 0;
  for (int q0 = c0; q0 < c1; q0 += UNR) {
    float4 xb[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) xb[u] = row4[min(q0 + u, n4 - 1)];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (q0 + u < c1) {
        const float xs[4] = {xb[u].x, xb[u].y, xb[u].z, xb[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t bb;
          if (weight(xs[e], bb) != 0 && bb == ph) ++mine;
        }
      }
  }
  uint32_t incl = mine;
  const int lane = tid & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, o, 64);
    if (lane >= o) incl += y;
  }
  __syncthreads();
  if (lane == 63) red32[tid >> 6] = incl;
  __syncthreads();
  uint32_t base = 0;
  for (int i = 0; i < (tid >> 6); ++i) base += red32[i];
  const uint32_t excl = base + incl - mine;
  if (mine && j >= excl && j < excl + mine) {
    int k = (int)(j - excl), pick = -1;
    for (int q0 = c0; q0 < c1 && pick < 0; q0 += UNR) {
      float4 xb[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) xb[u] = row4[min(q0 + u, n4 - 1)];
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        if (q0 + u < c1) {
          const float xs[4] = {xb[u].x, xb[u].y, xb[u].z, xb[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t bb;
            if (weight(xs[e], bb) != 0 && bb == ph) {
              if (k == 0 && pick < 0) pick = 4 * (q0 + u) + e;
              --k;
            }
          }
        }
    }
    out[r] = pick < 0 ? 0 : pick;
  }
}

hipError_t launch_sample_top_p(const float* logits, int rows, int vocab, const SampleArgs& p, int32_t* out,
                               hipStream_t st) {
  launch_kernel(sample_top_p_kernel, dim3(rows), dim3(kSampleThreads), 0, st, logits, vocab, p, out);
  return hipGetLastError();
}

}  // namespace cbd
