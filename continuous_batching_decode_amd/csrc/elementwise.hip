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

}  // namespace cbd
