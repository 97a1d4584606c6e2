// Row-wise kernels of the decode step: embedding gather (with the first
// norm's gain and sums of squares), RoPE at each row's own position + K/V
// append into its slab, greedy argmax, activation plane split, and slab
// scatter/gather for seeding and inspection.
//
// Position discipline (page "Batching", section 5): a row's position is read
// once per step from its metadata and used for both the query and the key
// rotation and for the slab slot the key is written to.
#include <mutex>

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

// Store the code of (key, dim d) of a K (kv = 0) or V region; lane = d within its group of 64, every
// lane of the wave calling. 4-bit K: dims d, d ^ 4 share a byte, written whole by the lane with bit 2
// clear; 4-bit V: keys kk, kk ^ 4 share a byte, so the nibble is set atomically.
template <int BITS>
CBD_DEVICE void store_code(uint8_t* base, int kv, int key, int d, int dh, uint32_t code, int lane) {
  if constexpr (BITS == 8) {
    base[kv == 0 ? kq_off(key, d, dh) : vq_off(key, d, dh)] = (uint8_t)code;
  } else {
    const uint32_t other = __shfl_xor(code, 4, 64);
    if (kv == 0) {
      if ((lane & 4) == 0) base[kq4_off(key, d, dh)] = (uint8_t)(code | (other << 4));
    } else {
      store_nibble(base + vq4_off(key, d, dh), (vslab_kk(key) >> 2) & 1, code);
    }
  }
}
template <int BITS>
CBD_DEVICE uint32_t load_code(const uint8_t* base, int kv, int key, int d, int dh) {
  if constexpr (BITS == 8) return base[kv == 0 ? kq_off(key, d, dh) : vq_off(key, d, dh)];
  const uint32_t b = kv == 0 ? base[kq4_off(key, d, dh)] : base[vq4_off(key, d, dh)];
  return (b >> (4 * (kv == 0 ? (d >> 2) & 1 : (vslab_kk(key) >> 2) & 1))) & 15u;
}

// The same for affine 8-bit slabs: queries rotate in place; each (KV head, group of 64 dims) of the
// row's k (rotated) and v is rounded to bf16 and quantized by one wave (lane = dim), as the
// quantizing append does.
template <int BITS>
__global__ __launch_bounds__(256) void rope_append_q8_kernel(float* qkv, int ld_qkv, const RowMeta* meta, int n_heads,
                                                             int n_kv_heads, int head_dim, int layer, uint8_t* arena,
                                                             const float2* rope_cs) {
  const int r = blockIdx.x;
  const RowMeta m = meta[r];
  const int half = head_dim >> 1;
  const float2* cs = rope_cs + (int64_t)m.pos * half;
  float* q = qkv + (int64_t)r * ld_qkv;
  const float* k = q + n_heads * head_dim;
  const float* v = k + n_kv_heads * head_dim;
  for (int idx = threadIdx.x; idx < n_heads * half; idx += 256) {
    const int hh = idx / half, i = idx - hh * half;
    float* x = q + hh * head_dim;
    const float2 c = cs[i];
    const float x1 = x[i], x2 = x[i + half];
    x[i] = x1 * c.x - x2 * c.y;
    x[i + half] = x2 * c.x + x1 * c.y;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ng = head_dim / kQGroup, units = 2 * n_kv_heads * ng;
  const int64_t region = (int64_t)(m.stride / 32) * q_block_bytes(head_dim, BITS);
  uint8_t* slab = arena + m.slab_off;
  for (int u = wave; u < units; u += 4) {
    const int kv = u / (n_kv_heads * ng), rem = u - kv * n_kv_heads * ng;
    const int j = rem / ng, gi = rem - j * ng, d = gi * kQGroup + lane;
    uint8_t* base = slab + ((int64_t)(layer * 2 + kv) * n_kv_heads + j) * region;
    float x;
    if (kv == 0) {
      const float* kx = k + j * head_dim;
      const int i = d < half ? d : d - half;
      const float2 c = cs[i];
      const float x1 = kx[i], x2 = kx[i + half];
      x = d < half ? x1 * c.x - x2 * c.y : x2 * c.x + x1 * c.y;
    } else {
      x = v[j * head_dim + d];
    }
    x = bf16_to_f32(f32_to_bf16(x));
    const float lo = -wave_max(-x), sc = q8_scale<BITS>(lo, wave_max(x));
    const uint32_t code = q8_code<BITS>(x, lo, sc);
    store_code<BITS>(base, kv, m.pos, d, head_dim, code, lane);
    if (lane == 0) *reinterpret_cast<float2*>(base + sbq_off(m.pos, gi, head_dim, BITS)) = float2{sc, lo};
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
                                                        int n_all, int t_off, int n_kv_heads, int head_dim,
                                                        const uint16_t* k_in,
                                                        const uint16_t* v_in, uint16_t* k_out, uint16_t* v_out) {
  const int t = blockIdx.x, l = blockIdx.y, kv = blockIdx.z;
  const int chunks = n_kv_heads * head_dim / 8;
  uint16_t* slab = reinterpret_cast<uint16_t*>(arena + slab_off);
  const int64_t region = (int64_t)stride * head_dim;
  const int64_t canon = ((int64_t)l * n_all + t_off + t) * n_kv_heads * head_dim;
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

// Affine 8-bit slabs: one wave per (token, layer, K or V, KV head, group of 64 dims), lane = dim.
template <int BITS>
__global__ __launch_bounds__(256) void slab_q8_kernel(uint8_t* arena, int64_t slab_off, int stride, int pos, int n_all,
                                                      int t_off, int n_kv_heads, int head_dim, const uint16_t* k_in,
                                                      const uint16_t* v_in, uint8_t* codes_out, float* sb_out) {
  const int t = blockIdx.x, l = blockIdx.y, kv = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ng = head_dim / kQGroup, units = n_kv_heads * ng;
  const int64_t region = (int64_t)(stride / 32) * q_block_bytes(head_dim, BITS);
  const int key = pos + t;
  for (int u = wave; u < units; u += 4) {
    const int j = u / ng, gi = u - j * ng, d = gi * kQGroup + lane;
    uint8_t* base = arena + slab_off + ((int64_t)(l * 2 + kv) * n_kv_heads + j) * region;
    float2* sbp = reinterpret_cast<float2*>(base + sbq_off(key, gi, head_dim, BITS));
    if (k_in) {
      const uint16_t* in = kv == 0 ? k_in : v_in;
      const float x = bf16_to_f32(in[(((int64_t)l * n_all + t_off + t) * n_kv_heads + j) * head_dim + d]);
      const float lo = -wave_max(-x), s = q8_scale<BITS>(lo, wave_max(x));
      store_code<BITS>(base, kv, key, d, head_dim, q8_code<BITS>(x, lo, s), lane);
      if (lane == 0) *sbp = float2{s, lo};
    } else {
      const int64_t o = (((int64_t)l * n_all + t_off + t) * 2 + kv) * n_kv_heads + j;
      codes_out[o * head_dim + d] = (uint8_t)load_code<BITS>(base, kv, key, d, head_dim);
      if (lane == 0) reinterpret_cast<float2*>(sb_out)[o * ng + gi] = *sbp;
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

hipError_t launch_rope_append_q8(float* qkv, int ld_qkv, const RowMeta* meta, int rows, int n_heads, int n_kv_heads,
                                 int head_dim, int layer, uint8_t* arena, const float* rope_cs, int bits,
                                 hipStream_t st) {
  if (head_dim % kQGroup || (bits != 8 && bits != 4)) return hipErrorInvalidValue;
  launch_kernel(bits == 8 ? rope_append_q8_kernel<8> : rope_append_q8_kernel<4>, dim3(rows), dim3(256), 0, st, qkv,
                ld_qkv, meta, n_heads, n_kv_heads, head_dim, layer, arena, reinterpret_cast<const float2*>(rope_cs));
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

hipError_t launch_slab_copy(uint8_t* arena, int64_t slab_off, int stride, int pos, int n, int n_all, int t_off,
                            int n_layers, int n_kv_heads, int head_dim, const uint16_t* k_in, const uint16_t* v_in,
                            uint16_t* k_out, uint16_t* v_out, hipStream_t st) {
  launch_kernel(slab_copy_kernel, dim3(n, n_layers, 2), dim3(256), 0, st, arena, slab_off, stride, pos, n_all, t_off,
                n_kv_heads, head_dim, k_in, v_in, k_out, v_out);
  return hipGetLastError();
}

hipError_t launch_slab_q8(uint8_t* arena, int64_t slab_off, int stride, int pos, int n, int n_all, int t_off,
                          int n_layers, int n_kv_heads, int head_dim, const uint16_t* k_in, const uint16_t* v_in,
                          uint8_t* codes_out, float* sb_out, int bits, hipStream_t st) {
  if (head_dim % kQGroup || stride % 32 || (bits != 8 && bits != 4)) return hipErrorInvalidValue;
  launch_kernel(bits == 8 ? slab_q8_kernel<8> : slab_q8_kernel<4>, dim3(n, n_layers, 2), dim3(256), 0, st, arena,
                slab_off, stride, pos, n_all, t_off, n_kv_heads, head_dim, k_in, v_in, codes_out, sb_out);
  return hipGetLastError();
}


// ============================================================================ seeded top-p sampling
// Row r: temperature T_r, nucleus mass p_r, draw from Philox4x64-10 with key (seed_r, 0) and counter
// (index_r, 0, 0, 0). T_r = 0 is greedy (lowest id among maxima). Otherwise e_i = exp(z_i - max z)
// with z = logit / T, in fixed point w_i = floor(e_i 2^40) (integer masses: every comparison below
// is exact and order-free). The nucleus is the shortest prefix of the ids ordered by e descending
// (ties: lower id first) whose mass reaches floor(p_r W), W = sum w; the token is the first of that
// order whose running mass exceeds floor(u M), M = nucleus mass, u the 24-bit draw. Both searches
// descend the bit patterns of e (order-preserving for positive floats) byte by byte. A row is cut
// into kSampleChunks chunks of consecutive ids, one workgroup each, over nine launches: chunk maxima;
// then the weights (kept as bit patterns in the workspace) with the chunk's mass and its histogram of
// top bytes, added into the row's histogram with integer atomics (order-free sums); then each level:
// every workgroup reads the row's histogram of the level decided last, picks the byte where the
// running mass from the top crosses the target, and adds its own chunk's histogram of the next byte
// inside that prefix. The last launch resolves the ties at the final pattern in id order over the
// chunks' counts (kept per chunk).
#ifndef CBD_SAMPLE_UNR
#define CBD_SAMPLE_UNR 8
#endif
namespace {
constexpr int kSampleThreads = 256;
constexpr int kSampleWaves = kSampleThreads / 64;

// Philox4x64-10 word 0 for counter (ctr, 0, 0, 0) and key (k0, 0)
CBD_DEVICE uint64_t philox_word0(uint64_t ctr, uint64_t k0) {
  uint64_t c0 = ctr, c1 = 0, c2 = 0, c3 = 0, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t h0 = __umul64hi(c0, 0xD2E7470EE14C6C93ull), l0 = c0 * 0xD2E7470EE14C6C93ull;
    const uint64_t h1 = __umul64hi(c2, 0xCA5A826395121157ull), l1 = c2 * 0xCA5A826395121157ull;
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

// fixed-point weight floor(e 2^40) of a bit pattern of e in [0, 1]: the mantissa shifted by the
// exponent (exact; 0 below 2^-40 and for the zero pattern)
CBD_DEVICE uint64_t fixed_of(uint32_t bits) {
  const int ex = (int)(bits >> 23);
  const uint64_t man = (uint64_t)((bits & 0x7FFFFFu) | 0x800000u);
  const int sh = ex - 110;  // e 2^40 = man 2^(ex - 127 - 23 + 40)
  return (ex == 0 || ex > 127) ? 0ull : sh >= 0 ? man << sh : (sh > -24 ? man >> (-sh) : 0ull);
}

template <typename T>
CBD_DEVICE T wg_sum(T v, T* red) {  // fixed order: lanes by xor tree, then the waves in order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  T s = 0;
  for (int i = 0; i < kSampleWaves; ++i) s += red[i];
  return s;
}

// per-row state carried between the launches (written by the row's first workgroup)
struct SampleState {
  uint64_t W, target, above_th, keep, wth, t, excess;
  uint32_t pre;   // bytes of the nucleus pattern decided so far
  uint32_t th, nt;
  uint32_t pre2;  // bytes of the sampled pattern decided so far
  uint64_t above, above2;
};
}  // namespace

SampleWs sample_ws_layout(uint8_t* base, int vocab) {
  SampleWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    uint8_t* q = base ? base + o : nullptr;
    o += (bytes + 255) / 256 * 256;
    return q;
  };
  w.bits = reinterpret_cast<uint32_t*>(take((size_t)64 * vocab * 4));
  w.pmax = reinterpret_cast<float*>(take((size_t)64 * kSampleChunks * 4));
  w.pidx = reinterpret_cast<int32_t*>(take((size_t)64 * kSampleChunks * 4));
  w.pw = reinterpret_cast<uint64_t*>(take((size_t)64 * kSampleChunks * 8));
  w.hist = reinterpret_cast<uint64_t*>(take((size_t)7 * 64 * kSampleChunks * 256 * 8));
  w.cnt = reinterpret_cast<uint32_t*>(take((size_t)2 * 64 * kSampleChunks * 256 * 4));
  w.state = take((size_t)64 * sizeof(SampleState));
  w.bytes = o;
  return w;
}

__global__ __launch_bounds__(kSampleThreads) void sample_phase_kernel(const float* logits, int vocab, SampleArgs p,
                                                                      SampleWs ws, int phase, int32_t* out) {
  __shared__ uint64_t hm[256];
  __shared__ uint32_t hc[256];
  __shared__ uint64_t red64[kSampleWaves];
  __shared__ float redf[kSampleWaves];
  __shared__ uint32_t red32[kSampleWaves];
  __shared__ uint32_t s_bin;
  __shared__ uint64_t s_above;
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  constexpr int C = kSampleChunks;   // chunks of a row (gridDim.x)
  constexpr int CS = kSampleChunks;  // slots per row in the workspace
  const float4* row4 = reinterpret_cast<const float4*>(logits + (int64_t)r * vocab);
  const int n4 = vocab >> 2;  // vocab % 4 == 0 (checked by the host)
  const int cs4 = (n4 + C - 1) / C;
  const int q0 = c * cs4, q1 = min(n4, q0 + cs4);  // this chunk's float4s
  uint32_t* bits = ws.bits + (int64_t)r * vocab;
  SampleState* stp = reinterpret_cast<SampleState*>(ws.state) + r;
  const float temp = p.temperature[r];
  const bool greedy = temp == 0.f;
  auto H = [&](int lv) { return ws.hist + ((int64_t)lv * 64 + r) * CS * 256; };  // [chunk][256]
  auto N = [&](int k) { return ws.cnt + ((int64_t)k * 64 + r) * CS * 256; };
  // the chunk's float4s q0 + tid + 256 i in increasing order, 8 loads in flight (clamped indices)
  constexpr int UNR = CBD_SAMPLE_UNR;
  auto each4 = [&](const uint4* src, auto&& visit) {
    for (int qa = q0 + tid; qa < q1; qa += UNR * kSampleThreads) {
      uint4 v[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) v[u] = src[min(qa + u * kSampleThreads, q1 - 1)];
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        if (qa + u * kSampleThreads < q1) visit(qa + u * kSampleThreads, v[u]);
    }
  };

  // From the row's histogram of one byte level (region `pre` of the `lv` bytes above), take off
  // the nucleus ties beyond `keep` where the boundary pattern lies in the region, and find the byte
  // where the running mass from the top, starting at `above`, crosses `target` (>= when ge, else >).
  auto decide = [&](const uint64_t* h, int lv, uint32_t pre, uint64_t above, uint64_t target, bool ge,
                    uint32_t cap_bits, uint64_t cap_excess, uint32_t& bin, uint64_t& above_out) {
    const int b = 255 - tid;  // thread t holds byte 255 - t: the scan runs from the top
    uint64_t m = h[b];        // the row's histogram (the chunks' ones were added into it)
    if (cap_excess && (lv == 0 || (cap_bits >> (32 - 8 * lv)) == pre) && ((cap_bits >> (24 - 8 * lv)) & 255) == (uint32_t)b)
      m -= cap_excess;
    uint64_t incl = m;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    __syncthreads();
    if (lane == 63) red64[tid >> 6] = incl;
    if (tid == 0) {
      s_bin = 0;  // (unreachable fallback: the lowest byte)
      s_above = above;
    }
    __syncthreads();
    for (int i = 0; i < (tid >> 6); ++i) incl += red64[i];
    const uint64_t a0 = above + incl - m, a1 = above + incl;
    const bool before = ge ? a0 >= target : a0 > target, after = ge ? a1 >= target : a1 > target;
    if (!before && after) {
      s_bin = (uint32_t)b;
      s_above = a0;
    }
    __syncthreads();
    bin = s_bin;
    above_out = s_above;
    __syncthreads();
  };
  // histogram of this chunk's byte at level lv over the patterns in region `pre` (weights > 0)
  auto build = [&](int lv, uint32_t pre, uint64_t* h_out, uint32_t* n_out) {
    for (int i = tid; i < 256; i += kSampleThreads) {
      hm[i] = 0;
      hc[i] = 0;
    }
    __syncthreads();
    const int sh = 24 - 8 * lv;
    each4(reinterpret_cast<const uint4*>(bits), [&](int, uint4 bb) {
      const uint32_t bs[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (bs[e] && (lv == 0 || (bs[e] >> (sh + 8)) == pre)) {
          const int bin = (bs[e] >> sh) & 255;
          atomicAdd(reinterpret_cast<unsigned long long*>(&hm[bin]), (unsigned long long)fixed_of(bs[e]));
          if (n_out) atomicAdd(&hc[bin], 1u);
        }
    });
    __syncthreads();
    for (int i = tid; i < 256; i += kSampleThreads) {  // masses: added into the row's histogram
      if (hm[i]) atomicAdd(reinterpret_cast<unsigned long long*>(&h_out[i]), (unsigned long long)hm[i]);
      if (n_out) n_out[c * 256 + i] = hc[i];
    }
  };

  if (phase == 0) {  // chunk maxima (greedy: the chunk's maximum and its lowest id)
    if (c == 0 && tid == 0) out[r] = 0;  // stands if no weight is positive
    if (c == 0)  // the row's histograms of every level start empty
      for (int i = tid; i < 7 * 256; i += kSampleThreads) H(i >> 8)[i & 255] = 0;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    const float inv_t = greedy ? 1.f : 1.f / temp;
    each4(reinterpret_cast<const uint4*>(row4), [&](int q, uint4 xb) {
      const float xs[4] = {__uint_as_float(xb.x), __uint_as_float(xb.y), __uint_as_float(xb.z), __uint_as_float(xb.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float z = greedy ? xs[e] : xs[e] * inv_t;
        if (z > best || (z == best && 4 * q + e < bi)) {
          best = z;
          bi = 4 * q + e;
        }
      }
    });
    const float m = wave_max(best);
    __syncthreads();
    if (lane == 0) redf[tid >> 6] = m;
    __syncthreads();
    float mm = redf[0];
    for (int i = 1; i < kSampleWaves; ++i) mm = fmaxf(mm, redf[i]);
    uint32_t cand = (best == mm) ? (uint32_t)bi : 0x7FFFFFFFu;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cand = min(cand, (uint32_t)__shfl_xor((int)cand, o, 64));
    __syncthreads();
    if (lane == 0) red32[tid >> 6] = cand;
    __syncthreads();
    if (tid == 0) {
      uint32_t bb = red32[0];
      for (int i = 1; i < kSampleWaves; ++i) bb = min(bb, red32[i]);
      ws.pmax[r * CS + c] = mm;
      ws.pidx[r * CS + c] = (int32_t)bb;
    }
    return;
  }
  if (greedy) {  // the lowest id among the chunks' maxima, in chunk order
    if (phase == 1 && c == 0 && tid == 0) {
      float best = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int k = 0; k < C; ++k) {
        const float v = ws.pmax[r * CS + k];
        const int i = ws.pidx[r * CS + k];
        if (i != 0x7FFFFFFF && (v > best || (v == best && i < bi))) {
          best = v;
          bi = i;
        }
      }
      out[r] = bi == 0x7FFFFFFF ? 0 : bi;  // every logit NaN: token 0
    }
    return;
  }

  if (phase == 1) {  // weights of the chunk, its mass and its top-byte histogram
    float mz = -INFINITY;
#pragma unroll
    for (int k = 0; k < CS; ++k) mz = fmaxf(mz, ws.pmax[r * CS + min(k, C - 1)]);
    const float inv_t = 1.f / temp;
    uint64_t tw = 0;
    each4(reinterpret_cast<const uint4*>(row4), [&](int q, uint4 xb) {
      const float xs[4] = {__uint_as_float(xb.x), __uint_as_float(xb.y), __uint_as_float(xb.z), __uint_as_float(xb.w)};
      uint32_t bs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ev = __expf(xs[e] * inv_t - mz);
        const uint32_t b = (ev == ev) ? __float_as_uint(ev) : 0u;  // NaN: weight 0
        const uint64_t w = fixed_of(b);
        bs[e] = w ? b : 0u;
        tw += w;
      }
      reinterpret_cast<uint4*>(bits)[q] = make_uint4(bs[0], bs[1], bs[2], bs[3]);
    });
    const uint64_t cw = wg_sum<uint64_t>(tw, red64);
    if (tid == 0) ws.pw[r * CS + c] = cw;
    __syncthreads();
    build(0, 0u, H(0), nullptr);
    return;
  }

  SampleState s = *stp;  // the decisions of the earlier launches
  if (phase == 2) {
    uint64_t W = 0;
#pragma unroll
    for (int k = 0; k < CS; ++k) {
      const uint64_t v = ws.pw[r * CS + min(k, C - 1)];
      W += k < C ? v : 0ull;
    }
    uint64_t target = (uint64_t)((double)p.top_p[r] * (double)W);
    if (target == 0) target = 1;
    uint32_t b0;
    uint64_t a0;
    decide(H(0), 0, 0u, 0ull, target, true, 0u, 0ull, b0, a0);
    build(1, b0, H(1), nullptr);
    if (c == 0 && tid == 0) {
      s.W = W;
      s.target = target;
      s.pre = b0;
      s.above = a0;
      *stp = s;
    }
    return;
  }
  if (phase == 3 || phase == 4) {  // nucleus pattern, bytes 1 and 2
    const int lv = phase - 2;
    uint32_t b;
    uint64_t a;
    decide(H(lv), lv, s.pre, s.above, s.target, true, 0u, 0ull, b, a);
    const uint32_t pre = (s.pre << 8) | b;
    build(lv + 1, pre, H(lv + 1), lv + 1 == 3 ? N(0) : nullptr);
    if (c == 0 && tid == 0) {
      s.pre = pre;
      s.above = a;
      *stp = s;
    }
    return;
  }
  if (phase == 5) {  // nucleus pattern byte 3: the boundary, the nucleus mass, the draw; sampled byte 0
    uint32_t b;
    uint64_t a;
    decide(H(3), 3, s.pre, s.above, s.target, true, 0u, 0ull, b, a);
    const uint32_t th = (s.pre << 8) | b;
    uint32_t nt = 0;
#pragma unroll
    for (int k = 0; k < CS; ++k) {
      const uint32_t v = N(0)[min(k, C - 1) * 256 + b];
      nt += k < C ? v : 0u;
    }
    const uint64_t wth = fixed_of(th);
    uint64_t keep = wth ? (s.target > a ? (s.target - a + wth - 1) / wth : 1) : nt;
    keep = keep < 1 ? 1 : (keep > nt ? nt : keep);
    const uint64_t M = a + keep * wth;
    const uint64_t u24 = philox_word0(p.index[r], p.seed[r]) >> 40;
    const uint64_t t = u24 * (M >> 24) + ((u24 * (M & 0xFFFFFFull)) >> 24);  // floor(u M), exact
    const uint64_t excess = (uint64_t)(nt - keep) * wth;
    uint32_t b2;
    uint64_t a2;
    decide(H(0), 0, 0u, 0ull, t, false, th, excess, b2, a2);
    build(1, b2, H(4), nullptr);  // byte 1 of the sampled pattern, kept as histogram 4
    if (c == 0 && tid == 0) {
      s.th = th;
      s.nt = nt;
      s.above_th = a;
      s.keep = keep;
      s.wth = wth;
      s.t = t;
      s.excess = excess;
      s.pre2 = b2;
      s.above2 = a2;
      *stp = s;
    }
    return;
  }
  if (phase == 6 || phase == 7) {  // sampled pattern, bytes 1 and 2
    const int lv = phase - 5;
    uint32_t b;
    uint64_t a;
    decide(H(3 + lv), lv, s.pre2, s.above2, s.t, false, s.th, s.excess, b, a);
    const uint32_t pre = (s.pre2 << 8) | b;
    build(lv + 1, pre, H(4 + lv), lv + 1 == 3 ? N(1) : nullptr);
    if (c == 0 && tid == 0) {
      s.pre2 = pre;
      s.above2 = a;
      *stp = s;
    }
    return;
  }
  // phase 8: sampled pattern byte 3, then the j-th id (ascending) among the tokens with it
  uint32_t b;
  uint64_t a;
  decide(H(6), 3, s.pre2, s.above2, s.t, false, s.th, s.excess, b, a);
  const uint32_t ph = (s.pre2 << 8) | b;
  const uint64_t wph = fixed_of(ph);
  uint32_t nph = 0, before = 0, here = 0;
#pragma unroll
  for (int k = 0; k < CS; ++k) {
    const uint32_t n = k < C ? N(1)[min(k, C - 1) * 256 + b] : 0u;
    nph += n;
    if (k < c) before += n;
    if (k == c) here = n;
  }
  uint64_t j = wph ? (s.t - a) / wph : 0;
  const uint64_t avail = ph == s.th ? s.keep : nph;
  if (j >= avail) j = avail ? avail - 1 : 0;
  if (here == 0 || j < before || j >= (uint64_t)before + here) return;  // (uniform over the workgroup)
  // this chunk holds it: per-thread counts over contiguous runs of float4s, an exclusive scan, the pick
  const int per = (q1 - q0 + kSampleThreads - 1) / kSampleThreads;
  const int t0 = q0 + tid * per, t1 = min(q1, t0 + per);
  uint32_t mine = 0;
  for (int q = t0; q < t1; ++q) {
    const uint4 bb = reinterpret_cast<const uint4*>(bits)[q];
    mine += (bb.x == ph) + (bb.y == ph) + (bb.z == ph) + (bb.w == ph);
  }
  uint32_t incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, o, 64);
    if (lane >= o) incl += y;
  }
  __syncthreads();
  if (lane == 63) red32[tid >> 6] = incl;
  __syncthreads();
  for (int i = 0; i < (tid >> 6); ++i) incl += red32[i];
  const uint32_t excl = incl - mine;
  const uint64_t k = j - before;
  if (mine && k >= excl && k < (uint64_t)excl + mine) {
    int left = (int)(k - excl);
    for (int q = t0; q < t1; ++q) {
      const uint4 bb = reinterpret_cast<const uint4*>(bits)[q];
      const uint32_t bs[4] = {bb.x, bb.y, bb.z, bb.w};
      for (int e = 0; e < 4; ++e)
        if (bs[e] == ph) {
          if (left == 0) {
            out[r] = 4 * q + e;
            return;
          }
          --left;
        }
    }
  }
}

hipError_t launch_sample_top_p(const float* logits, int rows, int vocab, const SampleArgs& p, const SampleWs& ws,
                               int32_t* out, hipStream_t st) {
  for (int phase = 0; phase <= 8; ++phase) {
    launch_kernel(sample_phase_kernel, dim3(kSampleChunks, rows), dim3(kSampleThreads), 0, st, logits, vocab, p, ws,
                  phase, out);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

}  // namespace cbd

// ---------------------------------------------------------------------------- scratch-free argmax
//
// cbd_greedy_argmax_noalloc: greedy_argmax without a context, for callers that cannot allocate
// device memory (code under stream capture, tight serving loops). Its kernel's segment partials and
// arrival counters live in `scratch`, a file-scope device array: one copy per GPU, loaded with the
// code object and held until the process ends. Host code reaches it only through the device address
// hipGetSymbolAddress returns for the current device (the array's name is a host-side stand-in),
// looked up once per device on the first call there. Every call on a GPU shares that GPU's array:
// calls that overlap on one GPU (several streams or threads) race.

namespace {
constexpr int kNoallocRows = 64;
constexpr size_t kNoallocPartBytes = (size_t)kNoallocRows * cbd::kArgmaxSegments * 2 * sizeof(float);
constexpr size_t kNoallocBytes = kNoallocPartBytes + kNoallocRows * sizeof(int32_t);
constexpr int kNoallocMaxDevices = 64;
static_assert(kNoallocPartBytes % 256 == 0, "counters start 256-byte aligned");

__global__ __launch_bounds__(64) void clear_counters_kernel(int32_t* counters, int n) {
  if ((int)threadIdx.x < n) counters[threadIdx.x] = 0;
}

std::mutex g_scratch_mu;
uint8_t* g_scratch_dev[kNoallocMaxDevices] = {};
}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoallocBytes];

extern "C" cbd_status cbd_greedy_argmax_noalloc(const float* logits_dev, int32_t rows, int32_t vocab,
                                                int32_t* tokens_dev, cbd_stream stream) {
  if (rows < 0 || rows > kNoallocRows)
    return cbd::record_error(CBD_E_INVAL, "cbd_greedy_argmax_noalloc: rows must be in 0..64 (scratch holds 64 rows)");
  if (rows == 0) return CBD_OK;
  if (vocab < 4 || vocab % 4 || vocab > (1 << 30))
    return cbd::record_error(CBD_E_INVAL, "cbd_greedy_argmax_noalloc: vocab must be a multiple of 4 in 4..2^30");
  if (!logits_dev || !tokens_dev || (reinterpret_cast<uintptr_t>(logits_dev) & 15))
    return cbd::record_error(CBD_E_INVAL, "cbd_greedy_argmax_noalloc: null or misaligned pointer");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoallocMaxDevices)
    return cbd::record_error(CBD_E_HIP, "cbd_greedy_argmax_noalloc: no current device");
  uint8_t* base;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return cbd::record_error(CBD_E_HIP, "cbd_greedy_argmax_noalloc: scratch address: %s", hipGetErrorString(e));
      g_scratch_dev[dev] = static_cast<uint8_t*>(p);
    }
    base = g_scratch_dev[dev];
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = reinterpret_cast<float*>(base);
  int32_t* counters = reinterpret_cast<int32_t*>(base + kNoallocPartBytes);
  // the counters of the previous call are zero when it completed; cleared anyway (a kernel, not a
  // memset node, so the call can be captured into a graph)
  cbd::launch_kernel(clear_counters_kernel, dim3(1), dim3(64), 0, st, counters, (int)rows);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = cbd::launch_argmax(logits_dev, rows, vocab, part, counters, tokens_dev, st);
  if (e != hipSuccess) return cbd::record_error(CBD_E_HIP, "cbd_greedy_argmax_noalloc: %s", hipGetErrorString(e));
  return CBD_OK;
}

