// Ragged per-sequence attention over persistent slabs.
//
// Page "Continuous Decode Batching - the transformer capture", section
// "decode_step_batch - paint-by-numbers" (delta 3): each query row reads keys
// and values only from its own slab and attends to [0..=t_s]. The same
// kernel serves the segmented prefill, where a token at segment-local
// position p attends to [0..=p] of its segment's slab (the page's
// block-diagonal causal shape, section "REVISED"), so no query ever reads
// another sequence's keys.
//
// One workgroup (4 waves) = one work item (query row, key range) x one KV
// head; the G = Hq/Hkv query heads sharing that KV head are processed
// together so every K/V tile is read once for all of them (GQA reuse).
// Keys are streamed in tiles of 64 through LDS with a running (max, sum)
// softmax in fp32. Long histories are split across items
// (flash-decoding style) and merged by attn_combine_kernel with the
// log-sum-exp rule.
#include "common.h"
#include "kernels.h"

namespace cbd {

namespace {
constexpr int TILE = 64;
}

template <int DH, int G>
__global__ __launch_bounds__(256) void attention_kernel(const float* qkv, int ld_qkv, const RowMeta* meta,
                                                        const AttnItem* items, int n_heads, int n_kv_heads, int layer,
                                                        const uint8_t* arena, uint16_t* out, int64_t out_plane,
                                                        int ld_out, float* part_o, float* part_ml) {
  constexpr int KROW = DH + 8;          // padded LDS row (elements) against bank conflicts
  constexpr int CH = DH / 8;            // 16-byte chunks per key row
  constexpr int QD = DH / 4;            // dims per thread in the score phase
  constexpr int DPAIRS = DH / 2;        // threads per key group in the PV phase
  constexpr int KGROUPS = 256 / DPAIRS;  // key groups in the PV phase
  constexpr int KPER = TILE / KGROUPS;   // keys per thread per tile in the PV phase
  __shared__ float qs[G][DH];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[TILE][KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[TILE][KROW];
  __shared__ float S[G][TILE];
  __shared__ float alpha_s[G];
  __shared__ float red[KGROUPS][G][DH];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const AttnItem it = items[blockIdx.x];
  const int j = blockIdx.y;
  const RowMeta m = meta[it.row];
  const float scale = 1.0f / sqrtf((float)DH);

  const float* q = qkv + (int64_t)it.row * ld_qkv + (int64_t)j * G * DH;
  for (int i = tid; i < G * DH; i += 256) qs[i / DH][i % DH] = q[i];

  const int64_t head_stride = (int64_t)m.cap * DH;
  const uint16_t* slab = reinterpret_cast<const uint16_t*>(arena + m.slab_off);
  const uint16_t* kbase = slab + ((int64_t)(layer * 2 + 0) * n_kv_heads + j) * head_stride;
  const uint16_t* vbase = slab + ((int64_t)(layer * 2 + 1) * n_kv_heads + j) * head_stride;

  float m_run = -INFINITY, l_run = 0.f;  // held by wave h for head h (h < G)
  float o[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) o[h][0] = o[h][1] = 0.f;

  const int dp = tid % DPAIRS, kg = tid / DPAIRS;

  for (int kb = it.k_begin; kb < it.k_end; kb += TILE) {
    __syncthreads();  // previous tile fully consumed
    for (int c = tid; c < TILE * CH; c += 256) {
      const int r = c / CH, col = (c % CH) * 8;
      const int key = kb + r;
      uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key < it.k_end) {
        kv = *reinterpret_cast<const uint4*>(kbase + (int64_t)key * DH + col);
        vv = *reinterpret_cast<const uint4*>(vbase + (int64_t)key * DH + col);
      }
      *reinterpret_cast<uint4*>(&Ks[r][col]) = kv;
      *reinterpret_cast<uint4*>(&Vs[r][col]) = vv;
    }
    __syncthreads();
    // scores: 4 threads per key, QD dims each
    {
      const int r = tid >> 2, qd = tid & 3;
      float part[G];
#pragma unroll
      for (int h = 0; h < G; ++h) part[h] = 0.f;
#pragma unroll
      for (int d8 = 0; d8 < QD; d8 += 8) {
        const uint4 kk = *reinterpret_cast<const uint4*>(&Ks[r][qd * QD + d8]);
        const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = bf16_to_f32(kw[e] & 0xFFFFu), k1 = bf16_to_f32(kw[e] >> 16);
#pragma unroll
          for (int h = 0; h < G; ++h)
            part[h] += qs[h][qd * QD + d8 + 2 * e] * k0 + qs[h][qd * QD + d8 + 2 * e + 1] * k1;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = part[h];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (qd == 0) S[h][r] = (kb + r < it.k_end) ? s * scale : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax: wave h owns head h
    if (wave < G) {
      const float s = S[wave][lane];
      const float m_new = fmaxf(m_run, wave_max(s));
      const float p = (s == -INFINITY) ? 0.f : __expf(s - m_new);
      const float alpha = __expf(m_run - m_new);
      l_run = l_run * alpha + wave_sum(p);
      m_run = m_new;
      S[wave][lane] = p;
      if (lane == 0) alpha_s[wave] = alpha;
    }
    __syncthreads();
    // P.V: thread owns dims (2dp, 2dp+1) of all G heads over KPER keys
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = alpha_s[h];
      o[h][0] *= a;
      o[h][1] *= a;
    }
#pragma unroll 4
    for (int kk = 0; kk < KPER; ++kk) {
      const int r = kg * KPER + kk;
      const uint32_t v2 = *reinterpret_cast<const uint32_t*>(&Vs[r][2 * dp]);
      const float v0 = bf16_to_f32(v2 & 0xFFFFu), v1 = bf16_to_f32(v2 >> 16);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = S[h][r];
        o[h][0] += p * v0;
        o[h][1] += p * v1;
      }
    }
  }
  // combine the key groups in a fixed order
#pragma unroll
  for (int h = 0; h < G; ++h) {
    red[kg][h][2 * dp] = o[h][0];
    red[kg][h][2 * dp + 1] = o[h][1];
  }
  __shared__ float ml_s[G][2];
  if (wave < G && lane == 0) {
    ml_s[wave][0] = m_run;
    ml_s[wave][1] = l_run;
  }
  __syncthreads();
  for (int i = tid; i < G * DH; i += 256) {
    const int h = i / DH, d = i % DH;
    float acc = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < KGROUPS; ++g2) acc += red[g2][h][d];
    const int head = j * G + h;
    if (it.part < 0) {
      const float v = acc / ml_s[h][1];
      const uint32_t hi = f32_to_bf16(v);
      const int64_t o = (int64_t)it.row * ld_out + head * DH + d;
      out[o] = (uint16_t)hi;
      out[o + out_plane] = (uint16_t)f32_to_bf16(v - bf16_to_f32(hi));
    } else {
      part_o[((int64_t)it.part * n_heads + head) * DH + d] = acc;
      if (d == 0) {
        part_ml[((int64_t)it.part * n_heads + head) * 2 + 0] = ml_s[h][0];
        part_ml[((int64_t)it.part * n_heads + head) * 2 + 1] = ml_s[h][1];
      }
    }
  }
}

// row_parts[row] = (first partial slot, count); count 0 = row written directly.
__global__ void attn_combine_kernel(const float* part_o, const float* part_ml, const int2* row_parts, int n_heads,
                                    int head_dim, uint16_t* out, int64_t out_plane, int ld_out) {
  const int row = blockIdx.x, head = blockIdx.y;
  const int2 rp = row_parts[row];
  if (rp.y == 0) return;
  float M = -INFINITY;
  for (int s = 0; s < rp.y; ++s) M = fmaxf(M, part_ml[((int64_t)(rp.x + s) * n_heads + head) * 2]);
  for (int d = threadIdx.x; d < head_dim; d += blockDim.x) {
    float acc = 0.f, l = 0.f;
    for (int s = 0; s < rp.y; ++s) {
      const int64_t slot = (int64_t)(rp.x + s) * n_heads + head;
      const float w = __expf(part_ml[slot * 2] - M);
      acc += w * part_o[slot * head_dim + d];
      l += w * part_ml[slot * 2 + 1];
    }
    const float v = acc / l;
    const uint32_t hi = f32_to_bf16(v);
    const int64_t o = (int64_t)row * ld_out + head * head_dim + d;
    out[o] = (uint16_t)hi;
    out[o + out_plane] = (uint16_t)f32_to_bf16(v - bf16_to_f32(hi));
  }
}

template <int DH>
static hipError_t launch_attn_dh(int G, dim3 grid, hipStream_t st, const float* qkv, int ld_qkv, const RowMeta* meta,
                                 const AttnItem* items, int n_heads, int n_kv_heads, int layer, const uint8_t* arena,
                                 uint16_t* out, int64_t out_plane, int ld_out, float* part_o, float* part_ml) {
  switch (G) {
    case 1:
      hipLaunchKernelGGL((attention_kernel<DH, 1>), grid, dim3(256), 0, st, qkv, ld_qkv, meta, items, n_heads,
                         n_kv_heads, layer, arena, out, out_plane, ld_out, part_o, part_ml);
      break;
    case 2:
      hipLaunchKernelGGL((attention_kernel<DH, 2>), grid, dim3(256), 0, st, qkv, ld_qkv, meta, items, n_heads,
                         n_kv_heads, layer, arena, out, out_plane, ld_out, part_o, part_ml);
      break;
    case 4:
      hipLaunchKernelGGL((attention_kernel<DH, 4>), grid, dim3(256), 0, st, qkv, ld_qkv, meta, items, n_heads,
                         n_kv_heads, layer, arena, out, out_plane, ld_out, part_o, part_ml);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const float* qkv, int ld_qkv, const RowMeta* meta, const AttnItem* items, int n_items,
                            int n_heads, int n_kv_heads, int head_dim, int layer, const uint8_t* arena,
                            uint16_t* out, int64_t out_plane, int ld_out, float* part_o, float* part_ml,
                            hipStream_t st) {
  const int G = n_heads / n_kv_heads;
  dim3 grid(n_items, n_kv_heads);
  if (head_dim == 128)
    return launch_attn_dh<128>(G, grid, st, qkv, ld_qkv, meta, items, n_heads, n_kv_heads, layer, arena, out,
                               out_plane, ld_out, part_o, part_ml);
  if (head_dim == 64)
    return launch_attn_dh<64>(G, grid, st, qkv, ld_qkv, meta, items, n_heads, n_kv_heads, layer, arena, out,
                              out_plane, ld_out, part_o, part_ml);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(const float* part_o, const float* part_ml, const int32_t* row_parts, int rows,
                               int n_heads, int head_dim, uint16_t* out, int64_t out_plane, int ld_out,
                               hipStream_t st) {
  hipLaunchKernelGGL(attn_combine_kernel, dim3(rows, n_heads), dim3(head_dim), 0, st, part_o, part_ml,
                     reinterpret_cast<const int2*>(row_parts), n_heads, head_dim, out, out_plane, ld_out);
  return hipGetLastError();
}

}  // namespace cbd
