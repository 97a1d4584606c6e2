// Row-wise kernels of the decode step: embedding gather + RMSNorm, RMSNorm,
// RoPE at each row's own position + K/V append into its slab, greedy argmax,
// and slab scatter/gather for seeding and inspection.
//
// Position discipline (page "Batching", section 5): a row's position is read
// once per step from its metadata and used for both the query and the key
// rotation and for the slab slot the key is written to.
#include "common.h"
#include "kernels.h"

namespace cbd {

namespace {

// Sum over a 256-thread block in a fixed order (deterministic).
CBD_DEVICE float block_sum_256(float v, float* scratch4) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) scratch4[wave] = v;
  __syncthreads();
  const float t = (scratch4[0] + scratch4[1]) + (scratch4[2] + scratch4[3]);
  __syncthreads();
  return t;
}

// xrow = bf16(row * inv_rms(row) * g) for an fp32 row (src_f32) or a bf16 row (src_bf16).
template <bool BF16_SRC>
CBD_DEVICE void norm_row_to_bf16(const void* src, int d, const uint16_t* gain, float eps, uint16_t* xrow,
                                 float* scratch4) {
  auto load4 = [&](int i) -> float4 {
    if (BF16_SRC) {
      const uint2 ev = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + i);
      return make_float4(bf16_to_f32(ev.x & 0xFFFFu), bf16_to_f32(ev.x >> 16), bf16_to_f32(ev.y & 0xFFFFu),
                         bf16_to_f32(ev.y >> 16));
    }
    return *reinterpret_cast<const float4*>(static_cast<const float*>(src) + i);
  };
  float ss = 0.f;
  for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
    const float4 v = load4(i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum_256(ss, scratch4);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
    const float4 v = load4(i);
    const uint2 gg = *reinterpret_cast<const uint2*>(gain + i);
    uint2 o;
    o.x = pack_bf16x2(v.x * inv * bf16_to_f32(gg.x & 0xFFFFu), v.y * inv * bf16_to_f32(gg.x >> 16));
    o.y = pack_bf16x2(v.z * inv * bf16_to_f32(gg.y & 0xFFFFu), v.w * inv * bf16_to_f32(gg.y >> 16));
    *reinterpret_cast<uint2*>(xrow + i) = o;
  }
}

}  // namespace

__global__ __launch_bounds__(256) void embed_norm_kernel(const int32_t* tokens, const uint16_t* embed, int vocab,
                                                         int d, const uint16_t* gain, float eps, float* h,
                                                         uint16_t* xn) {
  __shared__ float scratch[4];
  const int r = blockIdx.x;
  int tok = tokens[r];
  tok = tok < 0 ? 0 : (tok >= vocab ? vocab - 1 : tok);  // ids stay on the device: clamp out-of-range ids
  const uint16_t* e = embed + (int64_t)tok * d;
  float* hrow = h + (int64_t)r * d;
  for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
    const uint2 ev = *reinterpret_cast<const uint2*>(e + i);
    float4 v = make_float4(bf16_to_f32(ev.x & 0xFFFFu), bf16_to_f32(ev.x >> 16), bf16_to_f32(ev.y & 0xFFFFu),
                           bf16_to_f32(ev.y >> 16));
    *reinterpret_cast<float4*>(hrow + i) = v;
  }
  // the norm reads the embedding row again (not h) so no thread reads another thread's global writes
  norm_row_to_bf16<true>(e, d, gain, eps, xn + (int64_t)r * d, scratch);
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* h, const int32_t* row_idx, int d,
                                                      const uint16_t* gain, float eps, uint16_t* xn) {
  __shared__ float scratch[4];
  const int r = blockIdx.x;
  const int src = row_idx ? row_idx[r] : r;
  norm_row_to_bf16<false>(h + (int64_t)src * d, d, gain, eps, xn + (int64_t)r * d, scratch);
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
  const int64_t head_stride = (int64_t)m.cap * head_dim;
  uint16_t* kbase = slab + (int64_t)(layer * 2 + 0) * n_kv_heads * head_stride + (int64_t)m.pos * head_dim;
  uint16_t* vbase = slab + (int64_t)(layer * 2 + 1) * n_kv_heads * head_stride + (int64_t)m.pos * head_dim;
  for (int idx = threadIdx.x; idx < n_kv_heads * half; idx += 256) {
    const int j = idx / half, i = idx - j * half;
    const float* x = k + j * head_dim;
    const float2 c = cs[i];
    const float x1 = x[i], x2 = x[i + half];
    uint16_t* dst = kbase + j * head_stride;
    dst[i] = (uint16_t)f32_to_bf16(x1 * c.x - x2 * c.y);
    dst[i + half] = (uint16_t)f32_to_bf16(x2 * c.x + x1 * c.y);
  }
  for (int idx = threadIdx.x; idx < n_kv_heads * head_dim; idx += 256) {
    const int j = idx / head_dim, i = idx - j * head_dim;
    vbase[j * head_stride + i] = (uint16_t)f32_to_bf16(v[idx]);
  }
}

// Greedy argmax of one row per block: strict > keeps the first maximum a
// thread sees; across threads equal values resolve to the lower index.
__global__ __launch_bounds__(256) void argmax_kernel(const float* logits, int vocab, int32_t* out) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const int r = blockIdx.x;
  const float* row = logits + (int64_t)r * vocab;
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int v = threadIdx.x * 4; v < vocab; v += 256 * 4) {
    const float4 x = *reinterpret_cast<const float4*>(row + v);
    if (x.x > best || (bi == 0x7FFFFFFF && x.x == best)) { best = x.x; bi = v; }
    if (x.y > best) { best = x.y; bi = v + 1; }
    if (x.z > best) { best = x.z; bi = v + 2; }
    if (x.w > best) { best = x.w; bi = v + 3; }
  }
  sv[threadIdx.x] = best;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      const float ov = sv[threadIdx.x + s];
      const int oi = si[threadIdx.x + s];
      const float mv = sv[threadIdx.x];
      const int mi = si[threadIdx.x];
      if (ov > mv || (ov == mv && oi < mi)) { sv[threadIdx.x] = ov; si[threadIdx.x] = oi; }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[r] = si[0] == 0x7FFFFFFF ? 0 : si[0];
}

// canonical [L, n, Hkv, Dh] <-> slab [L][2][Hkv][cap][Dh] at positions [pos, pos+n); 16-byte moves
__global__ __launch_bounds__(256) void slab_copy_kernel(uint8_t* arena, int64_t slab_off, int cap, int pos, int n,
                                                        int n_kv_heads, int head_dim, const uint16_t* k_in,
                                                        const uint16_t* v_in, uint16_t* k_out, uint16_t* v_out) {
  const int t = blockIdx.x, l = blockIdx.y, kv = blockIdx.z;
  const int chunks = n_kv_heads * head_dim / 8;
  uint16_t* slab = reinterpret_cast<uint16_t*>(arena + slab_off);
  const int64_t head_stride = (int64_t)cap * head_dim;
  const int64_t canon = ((int64_t)l * n + t) * n_kv_heads * head_dim;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const int j = (c * 8) / head_dim, i = (c * 8) - j * head_dim;
    uint16_t* s = slab + (int64_t)(l * 2 + kv) * n_kv_heads * head_stride + j * head_stride +
                  (int64_t)(pos + t) * head_dim + i;
    if (k_in) {
      const uint16_t* src = (kv ? v_in : k_in) + canon + c * 8;
      *reinterpret_cast<uint4*>(s) = *reinterpret_cast<const uint4*>(src);
    } else {
      uint16_t* dst = (kv ? v_out : k_out) + canon + c * 8;
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(s);
    }
  }
}

hipError_t launch_embed_norm(const int32_t* tokens, int rows, const uint16_t* embed, int vocab, int d,
                             const uint16_t* gain, float eps, float* h, uint16_t* xn, hipStream_t st) {
  hipLaunchKernelGGL(embed_norm_kernel, dim3(rows), dim3(256), 0, st, tokens, embed, vocab, d, gain, eps, h, xn);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* h, const int32_t* row_idx, int rows, int d, const uint16_t* gain, float eps,
                          uint16_t* xn, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, st, h, row_idx, d, gain, eps, xn);
  return hipGetLastError();
}

hipError_t launch_rope_append(float* qkv, int ld_qkv, const RowMeta* meta, int rows, int n_heads, int n_kv_heads,
                              int head_dim, int layer, uint8_t* arena, const float* rope_cs, hipStream_t st) {
  hipLaunchKernelGGL(rope_append_kernel, dim3(rows), dim3(256), 0, st, qkv, ld_qkv, meta, n_heads, n_kv_heads,
                     head_dim, layer, arena, reinterpret_cast<const float2*>(rope_cs));
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int rows, int vocab, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(argmax_kernel, dim3(rows), dim3(256), 0, st, logits, vocab, out);
  return hipGetLastError();
}

hipError_t launch_slab_copy(uint8_t* arena, int64_t slab_off, int cap, int pos, int n, int n_layers, int n_kv_heads,
                            int head_dim, const uint16_t* k_in, const uint16_t* v_in, uint16_t* k_out,
                            uint16_t* v_out, hipStream_t st) {
  hipLaunchKernelGGL(slab_copy_kernel, dim3(n, n_layers, 2), dim3(256), 0, st, arena, slab_off, cap, pos, n,
                     n_kv_heads, head_dim, k_in, v_in, k_out, v_out);
  return hipGetLastError();
}

}  // namespace cbd
