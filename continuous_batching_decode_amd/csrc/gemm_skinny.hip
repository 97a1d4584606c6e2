// Batched weight-streaming product for the decode step and its prefill.
//
// y[b, n] = sum_k W[n, k] x[b, k] for up to 64 activation rows per column block.
// The page "Continuous Decode Batching - the transformer capture" (section
// "The throughput law") is the reason for the shape of this kernel: the
// weight read w is paid once per launch whatever the number of rows, so the
// kernel streams W from HBM exactly once with wide coalesced loads and every
// row of the batch rides on that single read.
//
// Mapping (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//  - A operand = 16 consecutive weight rows x 32 inputs (lane l holds row
//    l%16, inputs 8*(l/16)..+7). Weights live in the library's streaming
//    layout: each such 1 KB fragment is stored contiguously in lane order and
//    fragments run along K, so every wave load instruction reads 1 KB of
//    consecutive memory (DRAM-friendly, unlike 16 rows x 64 bytes of a
//    row-major matrix). Loads are double-buffered in registers.
//  - B operand = 16 activation rows x the same 32 inputs, read from LDS: the
//    workgroup stages each chunk of the activations once and its 4 waves
//    share it, so the vector-memory path carries (almost) only weights.
//  - A workgroup = 4 waves x RT subtiles of 16 weight rows. The input dim is
//    split over S workgroups when the matrix is too small to fill the chip;
//    their partial tiles go to a workspace and the last workgroup to finish
//    (an atomic arrival counter, reset by that workgroup) adds them in a
//    fixed order and runs the epilogue, so results are deterministic.
//  - NB column tiles of 16 cover up to 16*NB activation rows; padding rows
//    only affect padding outputs (an MFMA output column depends only on the
//    same column of B), which are never stored.
// Activations are carried as two bf16 planes, x = hi + lo with hi = bf16(x)
// and lo = bf16(x - hi), so the product keeps about 16 significant bits of x
// (two MFMAs per weight fragment; the products are exact in fp32).
//
// RMSNorm is folded in algebraically: the producer of x writes g * h (the
// gain applied, the 1/rms scale not) together with per-16-feature partial
// sums of squares of h; the consumer multiplies its fp32 accumulators by
// 1/sqrt(sum/d + eps) in the epilogue, since W (g * h / rms) = (W (g * h)) / rms.
//
// int4 weights (4-bit affine, groups of 64 inputs): codes are widened to the
// bf16 values 128+q with one and-or per pair and multiplied on the MFMA unit;
// the affine map is applied once per group and output:
//   sum_k x_k (s q_k + b) = s * sum_k x_k (128 + q_k) + (b - 128 s) * sum_k x_k,
// where sum_k x_k over the group comes from one more MFMA with an all-ones A.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace cbd {

namespace {

CBD_DEVICE bf16x8_t as_frag(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
CBD_DEVICE bf16x8_t as_frag(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// weights are read once per launch: non-temporal loads keep them from
// evicting the activations, partial tiles and K/V held in the caches
CBD_DEVICE u32x4_t load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

CBD_DEVICE bf16x8_t lds_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// 8 int4 codes of one packed word -> bf16 (128 + q) in input order.
CBD_DEVICE bf16x8_t widen_codes(uint32_t w) {
  uint4 r;
  r.x = (w & 0x000F000Fu) | 0x43004300u;
  r.y = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  r.z = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  r.w = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return as_frag(r);
}

CBD_DEVICE f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

CBD_DEVICE float silu_f(float g) { return g / (1.0f + __expf(-g)); }

CBD_DEVICE int seg_of(const SkinnyArgs& a, int grow) {
  return grow < a.seg_end[0] ? 0 : (grow < a.seg_end[1] ? 1 : 2);
}
CBD_DEVICE int seg_begin(const SkinnyArgs& a, int s) { return s == 0 ? 0 : a.seg_end[s - 1]; }

// 4 consecutive values -> hi/lo bf16 planes (8 bytes each)
CBD_DEVICE void store_split4(uint16_t* hi, uint16_t* lo, float v0, float v1, float v2, float v3) {
  const uint32_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1), h2 = f32_to_bf16(v2), h3 = f32_to_bf16(v3);
  uint2 H, L;
  H.x = h0 | (h1 << 16);
  H.y = h2 | (h3 << 16);
  L.x = f32_to_bf16(v0 - bf16_to_f32(h0)) | (f32_to_bf16(v1 - bf16_to_f32(h1)) << 16);
  L.y = f32_to_bf16(v2 - bf16_to_f32(h2)) | (f32_to_bf16(v3 - bf16_to_f32(h3)) << 16);
  *reinterpret_cast<uint2*>(hi) = H;
  *reinterpret_cast<uint2*>(lo) = L;
}

}  // namespace

// LDS bytes of one launch: activation chunk (2 planes) + norm partial sums.
// Pack a row-major bf16 matrix [N, K] into the streaming layout (N % 16 == 0, K % 32 == 0).
__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint16_t* src, int64_t N, int64_t K, uint16_t* dst) {
  const int64_t chunks = N * K / 8;
  const int64_t kfr = K / 32;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * 256) {
    const int64_t f = c >> 6;
    const int l = (int)(c & 63);
    const int64_t tr = f / kfr, tk = f - tr * kfr;
    const int64_t row = 16 * tr + (l & 15), col = 32 * tk + 8 * (l >> 4);
    *reinterpret_cast<uint4*>(dst + 8 * c) = *reinterpret_cast<const uint4*>(src + row * K + col);
  }
}

hipError_t launch_pack_bf16(const uint16_t* src, int64_t N, int64_t K, uint16_t* dst, hipStream_t st) {
  const int64_t chunks = N * K / 8;
  const int blocks = (int)std::min<int64_t>((chunks + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_bf16_kernel, dim3(blocks), dim3(256), 0, st, src, N, K, dst);
  return hipGetLastError();
}

size_t skinny_lds_bytes(int nb, int kc) { return (size_t)2 * 16 * nb * (kc + 8) * 2 + (size_t)16 * 16 * nb * 4; }

template <int RT, int NB, int EPI, int FMT, int UC>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(SkinnyArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int ROWS = 16 * NB;
  constexpr int NACC = RT * NB * 4;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int blk = blockIdx.x;
  const int split = blockIdx.y;
  const int S = gridDim.y;
  const int xblk = blockIdx.z;
  const int K = a.K;
  const int Kr = K / S;
  const int kbeg = split * Kr;
  const int KC = a.kc;
  const int XROW = KC + 8;  // padded LDS row (elements): consecutive rows start 16 bytes apart mod the bank width
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* norm_part = reinterpret_cast<float*>(smem + (size_t)2 * ROWS * XROW * 2);  // [16][ROWS]
  __shared__ int s_last;

  const int col0 = xblk * ROWS;
  const int rows_valid = min(ROWS, a.rows - col0);

  // weight-row subtiles of this wave
  int sub_row[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    if constexpr (EPI == EPI_SWIGLU) {  // RT == 2: the gate and up rows of the same 16 features
      const int f0 = blk * 64 + 16 * wave;
      sub_row[i] = i == 0 ? f0 : a.seg_end[0] + f0;
    } else {
      sub_row[i] = blk * 64 * RT + wave * 16 * RT + 16 * i;
    }
  }

  f32x4_t acc[RT][NB];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[i][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // stage activation chunk [kc0, kc0 + KC) of this block's rows into LDS
  auto stage_x = [&](int kc0) {
    __syncthreads();  // the previous chunk has been consumed
    const int per_row = KC / 8;
    // only the valid rows: padding rows of the LDS tile feed padding outputs only
    for (int idx = threadIdx.x; idx < 2 * rows_valid * per_row; idx += 256) {
      const int plane = idx / (rows_valid * per_row);
      const int rem = idx - plane * rows_valid * per_row;
      const int r = rem / per_row, c8 = rem - r * per_row;
      const int row = a.x_rows ? a.x_rows[col0 + r] : col0 + r;
      const uint16_t* src = a.x + (int64_t)plane * a.x_plane + (int64_t)row * a.ldx + kc0 + 8 * c8;
      *reinterpret_cast<uint4*>(xs + (plane * ROWS + r) * XROW + 8 * c8) = *reinterpret_cast<const uint4*>(src);
    }
    __syncthreads();
  };

  const int spc = KC / ((FMT == FMT_BF16 ? 32 : 128) * UC);  // k-steps per chunk
  const int total = Kr / ((FMT == FMT_BF16 ? 32 : 128) * UC);

  if constexpr (FMT == FMT_BF16) {
    // fragment (tile row tr, k-fragment tk) at ((tr * K/32) + tk) * 512 elements; lane l at 8*l
    const uint16_t* wr[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int s = seg_of(a, sub_row[i]);
      const int tr = (sub_row[i] - seg_begin(a, s)) >> 4;
      wr[i] = reinterpret_cast<const uint16_t*>(a.w[s]) + ((int64_t)tr * (K >> 5) + (kbeg >> 5)) * 512 + 8 * lane;
    }
    u32x4_t A0[UC][RT], A1[UC][RT];
    auto loadw = [&](u32x4_t (&A)[UC][RT], int st) {
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int i = 0; i < RT; ++i) A[u][i] = load_stream(wr[i] + (int64_t)(st * UC + u) * 512);
    };
    auto compute = [&](const u32x4_t (&A)[UC][RT], int st) {
      const int koff = ((st % spc) * UC) * 32 + 8 * g;
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          const bf16x8_t xh = lds_frag(xs + (16 * c + r16) * XROW + koff + 32 * u);
          const bf16x8_t xl = lds_frag(xs + (ROWS + 16 * c + r16) * XROW + koff + 32 * u);
#pragma unroll
          for (int i = 0; i < RT; ++i) {
            acc[i][c] = mfma(as_frag(A[u][i]), xh, acc[i][c]);
            acc[i][c] = mfma(as_frag(A[u][i]), xl, acc[i][c]);
          }
        }
    };
    loadw(A0, 0);
    if (total > 1) loadw(A1, 1);
    for (int st = 0; st < total; st += 2) {
      if (st % spc == 0) stage_x(kbeg + (st / spc) * KC);
      if (st > 0 && st + 1 < total) loadw(A1, st + 1);
      compute(A0, st);
      if (st + 1 < total) {
        if ((st + 1) % spc == 0) stage_x(kbeg + ((st + 1) / spc) * KC);
        if (st + 2 < total) loadw(A0, st + 2);
        compute(A1, st + 1);
      }
    }
  } else {
    // int4: 128 inputs per step; lane l (row l%16, group g = l/16) reads its 4 words of the block
    const uint32_t* wr[RT];
    const uint16_t* ar[RT];
    int seg_rows[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int s = seg_of(a, sub_row[i]);
      const int sb = seg_begin(a, s);
      const int tr = (sub_row[i] - sb) >> 4;
      wr[i] = reinterpret_cast<const uint32_t*>(a.w[s]) + ((int64_t)tr * (K >> 7) + (kbeg >> 7)) * 256 + 4 * lane;
      seg_rows[i] = a.seg_end[s] - sb;
      ar[i] = reinterpret_cast<const uint16_t*>(a.aux[s]) + (int64_t)(sub_row[i] - sb + 4 * g) * 2;
    }
    const uint4 ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8_t ones = as_frag(ones_u);
    for (int st = 0; st < total; ++st) {
      if (st % spc == 0) stage_x(kbeg + (st / spc) * KC);
      u32x4_t Wq[UC][RT];
      uint4 SB[UC][RT][2];
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int i = 0; i < RT; ++i) {
          Wq[u][i] = load_stream(wr[i] + (int64_t)(st * UC + u) * 256);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int grp = ((kbeg + (st * UC + u) * 128) >> 6) + h;
            SB[u][i][h] = *reinterpret_cast<const uint4*>(ar[i] + (int64_t)grp * seg_rows[i] * 2);
          }
        }
#pragma unroll
      for (int u = 0; u < UC; ++u) {
        const int kb = ((st % spc) * UC + u) * 128;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8_t X[2][NB][2];
          f32x4_t xsum[NB];
#pragma unroll
          for (int c = 0; c < NB; ++c) {
            f32x4_t t = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const int off = kb + 64 * h + 16 * g + 8 * jj;
              X[jj][c][0] = lds_frag(xs + (16 * c + r16) * XROW + off);
              X[jj][c][1] = lds_frag(xs + (ROWS + 16 * c + r16) * XROW + off);
              t = mfma(ones, X[jj][c][0], t);
              t = mfma(ones, X[jj][c][1], t);
            }
            xsum[c] = t;
          }
#pragma unroll
          for (int i = 0; i < RT; ++i) {
            const uint32_t w0 = h ? Wq[u][i][2] : Wq[u][i][0];
            const uint32_t w1 = h ? Wq[u][i][3] : Wq[u][i][1];
            const bf16x8_t A0 = widen_codes(w0), A1 = widen_codes(w1);
            const uint4 sb = SB[u][i][h];
            float sc[4], bc[4];
            const uint32_t pr[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sc[e] = bf16_to_f32(pr[e] & 0xFFFFu);
              bc[e] = bf16_to_f32(pr[e] >> 16) - 128.0f * sc[e];
            }
#pragma unroll
            for (int c = 0; c < NB; ++c) {
              f32x4_t t = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int p = 0; p < 2; ++p) {
                t = mfma(A0, X[0][c][p], t);
                t = mfma(A1, X[1][c][p], t);
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][c][e] += sc[e] * t[e] + bc[e] * xsum[c][e];
            }
          }
        }
      }
    }
  }

  // -- split-K: partial tiles to the workspace; the last workgroup of the row block adds them.
  (void)rows_valid;
  // Partial tiles and the arrival counter are written and read with agent-scope
  // atomic accesses, which the hardware performs at the level where all XCDs'
  // L2 caches agree; each wave waits for its stores to be acknowledged
  // (vmcnt 0) before the workgroup's arrival is counted. This avoids the full
  // L2 write-back and invalidate that a device-wide fence costs per workgroup.
  if (S > 1) {
    float* base = a.part + (int64_t)blk * S * 4 * NACC * 64;
    float* mine = base + ((int64_t)split * 4 + wave) * NACC * 64;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __hip_atomic_store(mine + ((i * NB + c) * 4 + e) * 64 + lane, acc[i][c][e], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are done
    __syncthreads();
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(a.counters + blk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c) acc[i][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
      const float* src = base + ((int64_t)s * 4 + wave) * NACC * 64;
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int c = 0; c < NB; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][c][e] += __hip_atomic_load(src + ((i * NB + c) * 4 + e) * 64 + lane, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.counters + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // 1/rms of each activation row from the producer's per-16-feature sums of squares, added in
  // 16 fixed groups (the same order in every workgroup and launch)
  float inv[NB];
  if (a.ss) {
    __syncthreads();  // LDS reuse: all waves are past their last activation read
    const int per = a.ss_tiles / 16;
    for (int i = threadIdx.x; i < 16 * ROWS; i += 256) {
      const int c = i % ROWS, grp = i / ROWS;
      float s = 0.f;
      if (c < rows_valid) {
        const int row = a.x_rows ? a.x_rows[col0 + c] : col0 + c;
        const float* p = a.ss + (int64_t)grp * per * a.ss_ld + row;
        for (int t = 0; t < per; ++t) s += p[(int64_t)t * a.ss_ld];
      }
      norm_part[grp * ROWS + c] = s;
    }
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    inv[c] = 1.f;
    if (a.ss) {
      float s = 0.f;
      for (int grp = 0; grp < 16; ++grp) s += norm_part[grp * ROWS + 16 * c + r16];
      inv[c] = 1.0f / sqrtf(s / a.norm_dim + a.eps);
    }
  }

  // epilogue: lane holds y[b = 16c + l%16][n = subtile + 4*(l/16) + e]
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int b = 16 * c + r16;
    const bool valid = b < rows_valid;
    const int64_t orow = (int64_t)(col0 + b) * a.ldo;
    if constexpr (EPI == EPI_SWIGLU) {
      static_assert(RT == 2, "gate and up subtiles");
      const int n = sub_row[0] + 4 * g;
      float m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) m[e] = silu_f(acc[0][c][e] * inv[c]) * (acc[1][c][e] * inv[c]);
      if (valid) store_split4(a.out_x + orow + n, a.out_x + a.out_plane + orow + n, m[0], m[1], m[2], m[3]);
    } else if constexpr (EPI == EPI_RESIDUAL) {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int n = sub_row[i] + 4 * g;
        float4 hn = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) {
          float4* p = reinterpret_cast<float4*>(a.out + orow + n);
          const float4 h = *p;
          hn = make_float4(h.x + acc[i][c][0], h.y + acc[i][c][1], h.z + acc[i][c][2], h.w + acc[i][c][3]);
          *p = hn;
          if (a.next_gain) {
            const uint2 gg = *reinterpret_cast<const uint2*>(a.next_gain + n);
            store_split4(a.out_x + orow + n, a.out_x + a.out_plane + orow + n, hn.x * bf16_to_f32(gg.x & 0xFFFFu),
                         hn.y * bf16_to_f32(gg.x >> 16), hn.z * bf16_to_f32(gg.y & 0xFFFFu),
                         hn.w * bf16_to_f32(gg.y >> 16));
          }
        }
        if (a.ss_out) {
          float s = hn.x * hn.x + hn.y * hn.y + hn.z * hn.z + hn.w * hn.w;
          s += __shfl_xor(s, 16, 64);
          s += __shfl_xor(s, 32, 64);
          if (valid && g == 0) a.ss_out[(int64_t)(sub_row[i] >> 4) * a.ss_out_ld + col0 + b] = s;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int n = sub_row[i] + 4 * g;
        if (valid)
          *reinterpret_cast<float4*>(a.out + orow + n) =
              make_float4(acc[i][c][0] * inv[c], acc[i][c][1] * inv[c], acc[i][c][2] * inv[c], acc[i][c][3] * inv[c]);
      }
    }
  }
}

// ----------------------------------------------------------------------------- launcher

bool skinny_shape_ok(int fmt, int K) { return fmt == FMT_INT4 ? K % 512 == 0 : K % 256 == 0; }

template <int RT, int EPI, int FMT, int UC>
static hipError_t launch_nb(const SkinnyArgs& a, int nb, dim3 grid, hipStream_t st) {
  const size_t lds = skinny_lds_bytes(nb, a.kc);
  switch (nb) {
    case 1: hipLaunchKernelGGL((skinny_gemm_kernel<RT, 1, EPI, FMT, UC>), grid, dim3(256), lds, st, a); break;
    case 2: hipLaunchKernelGGL((skinny_gemm_kernel<RT, 2, EPI, FMT, UC>), grid, dim3(256), lds, st, a); break;
    case 3: hipLaunchKernelGGL((skinny_gemm_kernel<RT, 3, EPI, FMT, UC>), grid, dim3(256), lds, st, a); break;
    default: hipLaunchKernelGGL((skinny_gemm_kernel<RT, 4, EPI, FMT, UC>), grid, dim3(256), lds, st, a); break;
  }
  return hipGetLastError();
}

// Plan of one launch: subtiles per wave, split of K, LDS chunk.
SkinnyPlan plan_skinny(int epi, int fmt, int N, int K, int rows, int x_blocks, int splits) {
  SkinnyPlan p{};
  const int per_block = x_blocks > 1 ? 64 : rows;
  p.nb = (per_block + 15) / 16;
  p.rt = (epi == EPI_SWIGLU || N % 128 == 0) ? 2 : 1;
  p.row_blocks = epi == EPI_SWIGLU ? N / 64 : N / (64 * p.rt);
  const int step = fmt == FMT_INT4 ? 128 : 32;
  p.uc = fmt == FMT_INT4 ? 1 : (p.nb > 2 ? 2 : 4);
  const int unit = step * p.uc;                    // one k-step of a wave
  const int kc_max = (960 / p.nb) / unit * unit;   // activation chunk: LDS stays within 64 KB
  if (splits > 0) {
    p.splits = splits;
  } else if (x_blocks > 1) {
    p.splits = 1;
  } else {
    // smallest split giving ~3 workgroups per CU, keeping >= 2 k-steps per wave and <= 16 partials
    p.splits = 1;
    for (int s = 2; s <= 16 && (long)p.row_blocks * p.splits < 768; ++s) {
      if (K % s || (K / s) % unit || K / s < 2 * unit) continue;
      p.splits = s;
    }
  }
  const int kr = K / p.splits;
  p.kc = unit;
  for (int kc = unit; kc <= std::min(kr, kc_max); kc += unit)
    if (kr % kc == 0) p.kc = kc;
  return p;
}

hipError_t launch_skinny_gemm(SkinnyArgs a, int epi, int fmt, int x_blocks, const SkinnyPlan& p, hipStream_t st) {
  if (p.splits < 1 || a.K % p.splits || (x_blocks > 1 && p.splits > 1)) return hipErrorInvalidValue;
  const int kr = a.K / p.splits;
  const int unit = (fmt == FMT_INT4 ? 128 : 32) * p.uc;
  if (kr % p.kc || p.kc % unit) return hipErrorInvalidValue;
  if (p.splits > 1 && (!a.part || !a.counters)) return hipErrorInvalidValue;
  a.kc = p.kc;
  const dim3 grid(p.row_blocks, p.splits, x_blocks);
  if (fmt == FMT_INT4) {
    if (epi == EPI_SWIGLU) return launch_nb<2, EPI_SWIGLU, FMT_INT4, 1>(a, p.nb, grid, st);
    if (p.rt == 1) {
      if (epi == EPI_RESIDUAL) return launch_nb<1, EPI_RESIDUAL, FMT_INT4, 1>(a, p.nb, grid, st);
      return launch_nb<1, EPI_STORE, FMT_INT4, 1>(a, p.nb, grid, st);
    }
    if (epi == EPI_RESIDUAL) return launch_nb<2, EPI_RESIDUAL, FMT_INT4, 1>(a, p.nb, grid, st);
    return launch_nb<2, EPI_STORE, FMT_INT4, 1>(a, p.nb, grid, st);
  }
  if (p.uc == 4) {
    if (epi == EPI_SWIGLU) return launch_nb<2, EPI_SWIGLU, FMT_BF16, 4>(a, p.nb, grid, st);
    if (p.rt == 1) {
      if (epi == EPI_RESIDUAL) return launch_nb<1, EPI_RESIDUAL, FMT_BF16, 4>(a, p.nb, grid, st);
      return launch_nb<1, EPI_STORE, FMT_BF16, 4>(a, p.nb, grid, st);
    }
    if (epi == EPI_RESIDUAL) return launch_nb<2, EPI_RESIDUAL, FMT_BF16, 4>(a, p.nb, grid, st);
    return launch_nb<2, EPI_STORE, FMT_BF16, 4>(a, p.nb, grid, st);
  }
  if (epi == EPI_SWIGLU) return launch_nb<2, EPI_SWIGLU, FMT_BF16, 2>(a, p.nb, grid, st);
  if (p.rt == 1) {
    if (epi == EPI_RESIDUAL) return launch_nb<1, EPI_RESIDUAL, FMT_BF16, 2>(a, p.nb, grid, st);
    return launch_nb<1, EPI_STORE, FMT_BF16, 2>(a, p.nb, grid, st);
  }
  if (epi == EPI_RESIDUAL) return launch_nb<2, EPI_RESIDUAL, FMT_BF16, 2>(a, p.nb, grid, st);
  return launch_nb<2, EPI_STORE, FMT_BF16, 2>(a, p.nb, grid, st);
}

}  // namespace cbd
