// Ragged per-sequence attention over persistent slabs.
//
// Page "Continuous Decode Batching - the transformer capture", section
// "decode_step_batch - paint-by-numbers": each query row rotates q and k at
// its own position t_s (delta 1), writes its new K/V into its own slab at
// t_s (delta 2), and attends only to [0..=t_s] of that slab (delta 3). The
// same kernel serves the segmented prefill (section "REVISED"), where a token
// at segment-local position p attends to [0..=p] of its segment's slab, so
// no query ever reads another sequence's keys (block-diagonal causal).
//
// One workgroup (4 waves) = one work item (query row, key range) x one KV
// head; the G = Hq/Hkv query heads sharing that KV head are processed
// together so every K/V tile is read once for all of them (GQA reuse). Keys
// stream through LDS in tiles of 64 with the next tile already in flight in
// registers; softmax is the running (max, sum) form in fp32. Long histories
// are split over several items (flash-decoding style); the last item of a
// (row, KV head) to finish merges the splits with the log-sum-exp rule.
#include "common.h"
#include "kernels.h"

namespace cbd {

namespace {
constexpr int TILE = 64;

CBD_DEVICE void store_split(uint16_t* hi, uint16_t* lo, float v) {
  const uint32_t h = f32_to_bf16(v);
  *hi = (uint16_t)h;
  *lo = (uint16_t)f32_to_bf16(v - bf16_to_f32(h));
}
}  // namespace

template <int DH, int G>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs a) {
  constexpr int KROW = DH + 8;           // padded LDS row (elements) against bank conflicts
  constexpr int CH = DH / 8;             // 16-byte chunks per key row
  constexpr int LOADS = TILE * CH / 256;  // 16-byte chunks per thread per tile (K and V each)
  constexpr int QD = DH / 4;             // dims per thread in the score phase
  constexpr int DPAIRS = DH / 2;         // threads per key group in the PV phase
  constexpr int KGROUPS = 256 / DPAIRS;   // key groups in the PV phase
  constexpr int KPER = TILE / KGROUPS;    // keys per thread per tile in the PV phase
  static_assert(LOADS >= 1, "tile too small");
  __shared__ float qs[G][DH];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[TILE][KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[TILE][KROW];
  __shared__ __attribute__((aligned(16))) uint16_t knew[DH], vnew[DH];
  __shared__ float S[G][TILE];
  __shared__ float alpha_s[G];
  __shared__ float red[KGROUPS][G][DH];
  __shared__ float ml_s[G][2];
  __shared__ int s_last;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const AttnItem it = a.items[blockIdx.x];
  const int j = blockIdx.y;
  const RowMeta m = a.meta[it.row];
  const int pos = m.pos;
  const float scale = 1.0f / sqrtf((float)DH);
  const int half = DH / 2;
  const float2* cs = a.rope_cs + (int64_t)pos * half;

  // queries of this KV group, rotated to pos when the projection left them unrotated
  const float* q = a.qkv + (int64_t)it.row * a.ld_qkv + (int64_t)j * G * DH;
  for (int i = tid; i < G * DH; i += 256) {
    const int h = i / DH, d = i % DH;
    float v = q[i];
    if (a.rope_q) {
      const int p = d < half ? d : d - half;
      const float2 c = cs[p];
      const float o = d < half ? q[i + half] : q[i - half];
      v = d < half ? v * c.x - o * c.y : v * c.x + o * c.y;
    }
    qs[h][d] = v;
  }

  const int64_t head_stride = (int64_t)m.cap * DH;
  uint16_t* slab = reinterpret_cast<uint16_t*>(a.arena + m.slab_off);
  uint16_t* kbase = slab + ((int64_t)(a.layer * 2 + 0) * a.n_kv_heads + j) * head_stride;
  uint16_t* vbase = slab + ((int64_t)(a.layer * 2 + 1) * a.n_kv_heads + j) * head_stride;

  // the item that ends at pos + 1 appends the new token's K/V (rotated, bf16) to the slab
  const bool appends = a.append && it.k_end == pos + 1;
  if (appends) {
    const float* kx = a.qkv + (int64_t)it.row * a.ld_qkv + (int64_t)a.n_heads * DH + (int64_t)j * DH;
    const float* vx = kx + (int64_t)a.n_kv_heads * DH;
    for (int d = tid; d < DH; d += 256) {
      const int p = d < half ? d : d - half;
      const float2 c = cs[p];
      const float o = d < half ? kx[d + half] : kx[d - half];
      const float kr = d < half ? kx[d] * c.x - o * c.y : kx[d] * c.x + o * c.y;
      const uint16_t kb = (uint16_t)f32_to_bf16(kr), vb = (uint16_t)f32_to_bf16(vx[d]);
      knew[d] = kb;
      vnew[d] = vb;
      kbase[(int64_t)pos * DH + d] = kb;
      vbase[(int64_t)pos * DH + d] = vb;
    }
  }

  float m_run = -INFINITY, l_run = 0.f;  // held by wave h for head h (h < G)
  float o[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) o[h][0] = o[h][1] = 0.f;
  const int dp = tid % DPAIRS, kg = tid / DPAIRS;

  // tile prefetch: keys at pos come from LDS when this item appended them
  const int key_lim = appends ? pos : it.k_end;  // keys read from the slab: [k_begin, key_lim)
  uint4 kreg[LOADS], vreg[LOADS];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int l = 0; l < LOADS; ++l) {
      const int c = tid + 256 * l;
      const int r = c / CH, col = (c % CH) * 8;
      const int key = kb + r;
      kreg[l] = vreg[l] = uint4{0u, 0u, 0u, 0u};
      if (key < key_lim) {
        kreg[l] = *reinterpret_cast<const uint4*>(kbase + (int64_t)key * DH + col);
        vreg[l] = *reinterpret_cast<const uint4*>(vbase + (int64_t)key * DH + col);
      }
    }
  };
  fetch(it.k_begin);
  for (int kb = it.k_begin; kb < it.k_end; kb += TILE) {
    __syncthreads();  // previous tile consumed (and the prologue's LDS writes done)
#pragma unroll
    for (int l = 0; l < LOADS; ++l) {
      const int c = tid + 256 * l;
      const int r = c / CH, col = (c % CH) * 8;
      if (appends && kb + r == pos) {
        kreg[l] = *reinterpret_cast<const uint4*>(knew + col);
        vreg[l] = *reinterpret_cast<const uint4*>(vnew + col);
      }
      *reinterpret_cast<uint4*>(&Ks[r][col]) = kreg[l];
      *reinterpret_cast<uint4*>(&Vs[r][col]) = vreg[l];
    }
    __syncthreads();
    if (kb + TILE < it.k_end) fetch(kb + TILE);  // next tile in flight during this one
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
      const float al = alpha_s[h];
      o[h][0] *= al;
      o[h][1] *= al;
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
  if (wave < G && lane == 0) {
    ml_s[wave][0] = m_run;
    ml_s[wave][1] = l_run;
  }
  __syncthreads();
  if (it.part < 0) {
    for (int i = tid; i < G * DH; i += 256) {
      const int h = i / DH, d = i % DH;
      float acc = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < KGROUPS; ++g2) acc += red[g2][h][d];
      const int64_t off = xfrag_off(it.row, (j * G + h) * DH + d, a.ld_out);
      store_split(a.out + off, a.out + a.out_plane + off, acc / ml_s[h][1]);
    }
    return;
  }
  // split item: publish the unnormalised partial; the last split of (row, KV head) merges.
  // Partials and the arrival counter use agent-scope atomic accesses (coherent across
  // the XCDs' L2 caches); stores are acknowledged (vmcnt 0) before arrival is counted.
  for (int i = tid; i < G * DH; i += 256) {
    const int h = i / DH, d = i % DH;
    float acc = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < KGROUPS; ++g2) acc += red[g2][h][d];
    const int64_t slot = (int64_t)it.part * a.n_heads + j * G + h;
    __hip_atomic_store(a.part_o + slot * DH + d, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d < 2) __hip_atomic_store(a.part_ml + slot * 2 + d, ml_s[h][d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  const int2 rp = a.row_parts[it.row];
  int32_t* counter = a.counters + (int64_t)it.row * a.n_kv_heads + j;
  if (tid == 0) s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == rp.y - 1;
  __syncthreads();
  if (!s_last) return;
  for (int i = tid; i < G * DH; i += 256) {
    const int h = i / DH, d = i % DH;
    float M = -INFINITY;
    for (int s = 0; s < rp.y; ++s) {
      const int64_t slot = (int64_t)(rp.x + s) * a.n_heads + j * G + h;
      M = fmaxf(M, __hip_atomic_load(a.part_ml + slot * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    float acc = 0.f, l = 0.f;
    for (int s = 0; s < rp.y; ++s) {
      const int64_t slot = (int64_t)(rp.x + s) * a.n_heads + j * G + h;
      const float w = __expf(__hip_atomic_load(a.part_ml + slot * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - M);
      acc += w * __hip_atomic_load(a.part_o + slot * DH + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      l += w * __hip_atomic_load(a.part_ml + slot * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int64_t off = xfrag_off(it.row, (j * G + h) * DH + d, a.ld_out);
    store_split(a.out + off, a.out + a.out_plane + off, acc / l);
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DH>
static hipError_t launch_attn_dh(int G, dim3 grid, hipStream_t st, const AttnArgs& a) {
  switch (G) {
    case 1: hipLaunchKernelGGL((attention_kernel<DH, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((attention_kernel<DH, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((attention_kernel<DH, 4>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int n_items, int head_dim, hipStream_t st) {
  const int G = a.n_heads / a.n_kv_heads;
  const dim3 grid(n_items, a.n_kv_heads);
  if (head_dim == 128) return launch_attn_dh<128>(G, grid, st, a);
  if (head_dim == 64) return launch_attn_dh<64>(G, grid, st, a);
  return hipErrorInvalidValue;
}

}  // namespace cbd
