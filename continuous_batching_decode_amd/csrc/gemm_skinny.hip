// Batched weight-streaming product for the decode step and its prefill.
//
// y[b, n] = sum_k W[n, k] x[b, k] for up to 64 activation rows per column block.
// The page "Continuous Decode Batching - the transformer capture" (section
// "The throughput law") is the reason for the shape of these kernels: the
// weight read w is paid once per launch whatever the number of rows, so they
// stream W from HBM exactly once with wide sequential loads and every row of
// the batch rides on that single read.
//
// Operands (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//  - A = 16 weight rows x 32 inputs (lane l: row l%16, inputs 8*(l/16)..+7).
//    Weights live in the streaming layout: each such 1 KB fragment is stored
//    contiguously in lane order and fragments run along K, so every wave load
//    instruction reads 1 KB of consecutive memory.
//  - B = 16 activation rows x the same 32 inputs, from activations stored
//    fragment-major the same way (xfrag_off).
//  - NB column tiles of 16 cover up to 16*NB activation rows; padding rows
//    only affect padding outputs (an MFMA output column depends only on the
//    same column of B), which are never stored.
// Two ways to cut a launch:
//  - k split (small matrices): one tile of 16*RT weight rows per workgroup;
//    its waves each stream a contiguous slice of K (double-buffered loads,
//    activations straight from L2) and add their partial sums through LDS in
//    a fixed order. No workgroup waits on another.
//  - row split (large matrices, and every prefill): 4 waves x RT subtiles of
//    16 rows share activation chunks staged once in LDS. If K must also be
//    split over workgroups, the partial tiles go to a workspace and the last
//    workgroup to arrive (agent-scope atomic counter, reset by it) adds them
//    in a fixed order. Results are deterministic either way.
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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace cbd {

namespace {

CBD_DEVICE bf16x8_t load_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// Constants of the int4 inner loops held in registers: gfx9 VALU instructions with three operands
// take no literal, so with the constants in registers widening a code pair and unpacking a (scale,
// bias) half are one instruction each (v_and_or_b32, v_and_b32).
struct Int4Consts {
  uint32_t bf16_128;  // 0x43004300: the bf16 pattern of 128 in both halves
  uint32_t pair_mask; // 0x000F000F: one code in each half
  uint32_t hi_mask;   // 0xFFFF0000
  CBD_DEVICE static Int4Consts make() {
    Int4Consts k{0x43004300u, 0x000F000Fu, 0xFFFF0000u};
    asm volatile("" : "+v"(k.bf16_128), "+v"(k.pair_mask), "+v"(k.hi_mask));
    return k;
  }
};

// 8 int4 codes of one packed word -> bf16 (128 + q) in input order.
CBD_DEVICE bf16x8_t widen_codes(uint32_t w, const Int4Consts& k) {
  u32x4_t r;
  r[0] = (w & k.pair_mask) | k.bf16_128;
  r[1] = ((w >> 4) & k.pair_mask) | k.bf16_128;
  r[2] = ((w >> 8) & k.pair_mask) | k.bf16_128;
  r[3] = ((w >> 12) & k.pair_mask) | k.bf16_128;
  return as_frag(r);
}

CBD_DEVICE float silu_f(float g) { return g / (1.0f + __expf(-g)); }

CBD_DEVICE int seg_of(const SkinnyArgs& a, int grow) {
  return grow < a.seg_end[0] ? 0 : (grow < a.seg_end[1] ? 1 : 2);
}
CBD_DEVICE int seg_begin(const SkinnyArgs& a, int s) { return s == 0 ? 0 : a.seg_end[s - 1]; }

// 4 consecutive inputs k..k+3 (k % 4 == 0) of one row -> hi/lo planes (8 bytes each)
CBD_DEVICE void store_split4(uint16_t* hi, uint16_t* lo, float v0, float v1, float v2, float v3) {
  uint2 H, L;
  H.x = pack_bf16x2(v0, v1);
  H.y = pack_bf16x2(v2, v3);
  L.x = pack_bf16x2(v0 - bf16_to_f32(H.x & 0xFFFFu), v1 - bf16_to_f32(H.x >> 16));
  L.y = pack_bf16x2(v2 - bf16_to_f32(H.y & 0xFFFFu), v3 - bf16_to_f32(H.y >> 16));
  *reinterpret_cast<uint2*>(hi) = H;
  *reinterpret_cast<uint2*>(lo) = L;
}

// First row of weight subtile i of tile t (16*RT consecutive rows, or for SwiGLU the gate and up
// rows of the same 16 features).
template <int RT, int EPI>
CBD_DEVICE int subtile_row(const SkinnyArgs& a, int t, int i) {
  if constexpr (EPI == EPI_SWIGLU) {  // RT/2 gate subtiles, then the up subtiles of the same features
    constexpr int H = RT / 2;
    return i < H ? 16 * H * t + 16 * i : a.seg_end[0] + 16 * H * t + 16 * (i - H);
  }
  return 16 * RT * t + 16 * i;
}

// Weight pointers (lane offset included) of the RT subtiles at input k0.
template <int RT, int FMT>
CBD_DEVICE void weight_ptrs(const SkinnyArgs& a, const int (&sub_row)[RT], int K, int k0, int lane,
                            const void* (&wr)[RT]) {
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int s = seg_of(a, sub_row[i]);
    const int tr = (sub_row[i] - seg_begin(a, s)) >> 4;
    if constexpr (FMT == FMT_BF16)
      wr[i] = reinterpret_cast<const uint16_t*>(a.w[s]) + ((int64_t)tr * (K >> 5) + (k0 >> 5)) * 512 + 8 * lane;
    else
      wr[i] = reinterpret_cast<const uint32_t*>(a.w[s]) + ((int64_t)tr * (K >> 7) + (k0 >> 7)) * 256 + 4 * lane;
  }
}

// 1/rms of each activation row of the block from the producer's per-16-feature sums of squares,
// added in 16 fixed groups (same order in every workgroup and launch). All threads take part;
// norm_part is [16][ROWS] floats of LDS.
template <int ROWS>
CBD_DEVICE void norm_partials(const SkinnyArgs& a, int col0, int rows_valid, float* norm_part) {
  const int per = a.ss_tiles / 16;
  for (int i = threadIdx.x; i < 16 * ROWS; i += blockDim.x) {
    const int c = i % ROWS, grp = i / ROWS;
    float s = 0.f;
    if (c < rows_valid) {
      const float* p = a.ss + (int64_t)grp * per * a.ss_ld + col0 + c;
      for (int t = 0; t < per; ++t) s += p[(int64_t)t * a.ss_ld];
    }
    norm_part[grp * ROWS + c] = s;
  }
}

// norm_part may hold nq sets of [16][ROWS] partials (set-major): each group adds its sets in
// order, then the 16 group sums are added in order. The 16 reads of a set are issued together (one
// LDS wait per set, not one per partial).
template <int ROWS>
CBD_DEVICE float norm_inv(const SkinnyArgs& a, const float* norm_part, int col, int nq) {
  float gs[16];
#pragma unroll
  for (int grp = 0; grp < 16; ++grp) gs[grp] = 0.f;
  for (int q = 0; q < nq; ++q) {
    float v[16];
#pragma unroll
    for (int grp = 0; grp < 16; ++grp) v[grp] = norm_part[(q * 16 + grp) * ROWS + col];
#pragma unroll
    for (int grp = 0; grp < 16; ++grp) gs[grp] += v[grp];
  }
  float s = 0.f;
#pragma unroll
  for (int grp = 0; grp < 16; ++grp) s += gs[grp];
  return 1.0f / sqrtf(s / a.norm_dim + a.eps);
}

// Epilogue of one wave. Lane l holds the products of column l%16 of each 8-row group c, rows
// n = subtile + 4*(l/16) + e: columns 0..7 are the hi parts of rows 8c + 0..7, columns 8..15 the lo
// parts. Adding lanes l and l^8 gives y[b = 8c + l%8][n] in both; lanes with l & 8 clear store it.
template <int RT, int NB, int EPI>
CBD_DEVICE void epilogue(const SkinnyArgs& a, f32x4_t (&acc)[RT][NB], const int (&sub_row)[RT], int col0,
                         int rows_valid, const float (&inv)[NB], int lane, const float4 (*hpre)[RT][NB]) {
  const int g = lane >> 4;
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int c = 0; c < NB; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][c][e] += __shfl_xor(acc[i][c][e], 8, 64);
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int b = 8 * c + (lane & 7);
    const bool valid = (lane & 8) == 0 && b < rows_valid;
    const int row = col0 + b;
    if constexpr (EPI == EPI_SWIGLU) {
      static_assert(RT % 2 == 0, "gate subtiles then their up subtiles");
#pragma unroll
      for (int i = 0; i < RT / 2; ++i) {
        const int n = sub_row[i] + 4 * g;
        float m[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = silu_f(acc[i][c][e] * inv[c]) * (acc[i + RT / 2][c][e] * inv[c]);
        if (valid) {
          const int64_t o = xfrag_off(row, n, a.N);
          store_split4(a.out_x + o, a.out_x + a.out_plane + o, m[0], m[1], m[2], m[3]);
        }
      }
    } else if constexpr (EPI == EPI_RESIDUAL) {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int n = sub_row[i] + 4 * g;
        float4 hn = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) {
          float4* p = reinterpret_cast<float4*>(a.out + (int64_t)row * a.ldo + n);
          const float4 h = hpre ? (*hpre)[i][c] : *p;
          hn = make_float4(h.x + acc[i][c][0], h.y + acc[i][c][1], h.z + acc[i][c][2], h.w + acc[i][c][3]);
          *p = hn;
          if (a.next_gain) {
            const uint2 gg = *reinterpret_cast<const uint2*>(a.next_gain + n);
            const int64_t o = xfrag_off(row, n, a.N);
            store_split4(a.out_x + o, a.out_x + a.out_plane + o, hn.x * bf16_to_f32(gg.x & 0xFFFFu),
                         hn.y * bf16_to_f32(gg.x >> 16), hn.z * bf16_to_f32(gg.y & 0xFFFFu),
                         hn.w * bf16_to_f32(gg.y >> 16));
          }
        }
        if (a.ss_out) {
          float s = hn.x * hn.x + hn.y * hn.y + hn.z * hn.z + hn.w * hn.w;
          s += __shfl_xor(s, 16, 64);
          s += __shfl_xor(s, 32, 64);
          if (valid && g == 0) a.ss_out[(int64_t)(sub_row[i] >> 4) * a.ss_out_ld + row] = s;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int n = sub_row[i] + 4 * g;
        if (valid)
          *reinterpret_cast<float4*>(a.out + (int64_t)row * a.ldo + n) =
              make_float4(acc[i][c][0] * inv[c], acc[i][c][1] * inv[c], acc[i][c][2] * inv[c], acc[i][c][3] * inv[c]);
      }
    }
  }
}

// int4 contribution of one 128-input block (4 k-fragments; fragments 0,1 form one group of 64,
// fragments 2,3 the next). X[j][c] = activation fragment j of 8-row group c (hi and lo columns).
template <int RT, int NB>
CBD_DEVICE void int4_block(f32x4_t (&acc)[RT][NB], const u32x4_t (&Wq)[RT], const uint4 (&SB)[RT][2],
                           const bf16x8_t (&X)[4][NB], const Int4Consts& k) {
  const u32x4_t ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = as_frag(ones_u);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4_t xsum[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      f32x4_t t = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) t = mfma(ones, X[2 * h + jj][c], t);
      xsum[c] = t;
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const bf16x8_t A0 = widen_codes(Wq[i][2 * h], k), A1 = widen_codes(Wq[i][2 * h + 1], k);
      const uint4 sb = SB[i][h];
      float sc[4], bc[4];
      const uint32_t pr[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // (scale, bias) as bf16 halves: scale = low half, bias = high half
        sc[e] = __uint_as_float(pr[e] << 16);
        bc[e] = fmaf(-128.0f, sc[e], __uint_as_float(pr[e] & k.hi_mask));
      }
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        f32x4_t t = f32x4_t{0.f, 0.f, 0.f, 0.f};
        t = mfma(A0, X[2 * h][c], t);
        t = mfma(A1, X[2 * h + 1][c], t);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][c][e] = fmaf(bc[e], xsum[c][e], fmaf(sc[e], t[e], acc[i][c][e]));
      }
    }
  }
}

// Where the scale/bias pairs of output rows 4g..4g+3 of each subtile are: group j of subtile i at
// p[i] + j * stride[i] (bf16 elements). Computed once per wave, before the stream: the segment
// lookup indexes the kernel arguments dynamically, which the compiler serves with scalar memory
// loads and a wait, so it stays out of the loop.
template <int RT>
struct ScaleRows {
  const uint16_t* p[RT];
  uint32_t stride[RT];  // (a table holds K/64 x N pairs: element offsets fit 32 bits)
};
template <int RT>
CBD_DEVICE ScaleRows<RT> scale_rows(const SkinnyArgs& a, const int (&sub_row)[RT], int g) {
  ScaleRows<RT> r;
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int s = seg_of(a, sub_row[i]);
    const int sb = seg_begin(a, s);
    r.p[i] = reinterpret_cast<const uint16_t*>(a.aux[s]) + (int64_t)(sub_row[i] - sb + 4 * g) * 2;
    r.stride[i] = (uint32_t)(a.seg_end[s] - sb) * 2u;
  }
  return r;
}
// scale/bias pairs of groups (k0/64, k0/64 + 1)
template <int RT>
CBD_DEVICE void load_scales(const ScaleRows<RT>& r, int k0, uint4 (&SB)[RT][2]) {
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      SB[i][h] = *reinterpret_cast<const uint4*>(r.p[i] + (uint32_t)((k0 >> 6) + h) * r.stride[i]);
}

}  // namespace

// ============================================================================ k split

// Build options for comparing vector-ALU inner products with the matrix cores at small batches:
// CBD_VALU_ROWS = n > 0 makes the bf16 k-split kernel with one 8-row group use fp32 FMAs whenever
// the batch has at most n rows, with CBD_VALU_DEPTH 32-input chunks in flight per wave. Off (0) by
// default: the matrix-core path measured faster at every batch of 1..4 rows.
#ifndef CBD_VALU_ROWS
#define CBD_VALU_ROWS 0
#endif
#ifndef CBD_VALU_DEPTH
#define CBD_VALU_DEPTH 4
#endif
constexpr int VALU_ROWS = CBD_VALU_ROWS;
constexpr int VALU_DEPTH = CBD_VALU_DEPTH;
static_assert(VALU_ROWS >= 0 && VALU_ROWS <= 8, "at most one 8-row group");

// Largest workgroup an instantiation is compiled for: 16 waves leave 128 registers per lane, enough
// for one subtile and one column tile; int4 with two row groups gets 4 waves (its stages hold the
// codes, their scales and 8 activation fragments); the others get 8 waves (256 registers).
template <int RT, int NB, int EPI, int FMT, int UC>
__global__ __launch_bounds__(((RT == 1 && NB == 1) ? 1024 : (FMT == FMT_INT4 && NB > 1) ? 256 : 512)) void
ksplit_gemm_kernel(SkinnyArgs a, int splits, int split_from) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int ROWS = 8 * NB;  // activation rows: NB groups of 8
  constexpr int NACC = RT * NB * 4;
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // workgroup (tile, split) takes inputs [split K/splits, (split + 1) K/splits), its waves a
  // contiguous 1/nw of that range each
  // Tiles below split_from take one workgroup each (the whole K); the others take `splits`
  // workgroups, so that the work per compute unit evens out when the tiles are not a whole
  // multiple of the units (ns: this workgroup's split count).
  int tile, split, ns;
  if ((int)blockIdx.x < split_from) {
    tile = blockIdx.x, split = 0, ns = 1;
  } else {
    const int r = blockIdx.x - split_from;
    tile = split_from + r / splits, split = r - (r / splits) * splits, ns = splits;
  }
  const int xblk = blockIdx.y;
  const int K = a.K, kw = K / (nw * ns), k0 = split * (K / ns) + wave * kw;
  const int col0 = xblk * ROWS;
  const int rows_valid = min(ROWS, a.rows - col0);
  float* red = reinterpret_cast<float*>(smem);              // [nw-1][NACC][64]
  float* norm_part = red + (size_t)(nw - 1) * NACC * 64;    // [16][ROWS]

  int sub_row[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) sub_row[i] = subtile_row<RT, EPI>(a, tile, i);
  const void* wr[RT];
  weight_ptrs<RT, FMT>(a, sub_row, K, k0, lane, wr);
  // activation fragment pointers at k0 for each 8-row group
  const uint16_t* xr[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) xr[c] = a.x + ((int64_t)((col0 >> 3) + c) * (K >> 5) + (k0 >> 5)) * 512 + 8 * lane;

  f32x4_t acc[RT][NB];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[i][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The epilogue's inputs that do not depend on the product are requested before the weights, so
  // their latency hides behind the stream. First the norm's per-16-feature sums of squares: the 16
  // groups x ROWS rows are split over nq thread sets, each adding ss_cnt consecutive partials in
  // order.
  constexpr int SSMAX = NB >= 2 ? 16 : 8;  // partials per thread (8: two thread sets per item at NB = 1)
  const int ss_per = a.ss ? a.ss_tiles / 16 : 0;
  int nq = 1;
  while (2 * nq * 16 * ROWS <= (int)blockDim.x && ss_per % (2 * nq) == 0) nq *= 2;
  const int ss_cnt = ss_per / nq;
  // (every one of the 16 x ROWS items needs a thread of its own)
  const bool ss_early = a.ss && ss_cnt <= SSMAX && (int)blockDim.x >= 16 * ROWS;
  const int ss_item = threadIdx.x % (16 * ROWS), ss_q = threadIdx.x / (16 * ROWS);
  const bool ss_mine = ss_early && ss_q < nq && (ss_item % ROWS) < rows_valid;
  // The loads are unconditional inside the (uniform) norm branch: threads without an item, and
  // partials past ss_cnt, reread valid ones that the sum skips. (The compiler would otherwise start
  // the sum next to the loads, waiting for them before any weight is requested.)
  float ssv[SSMAX];
  if (ss_early) {
    const float* p = a.ss + (ss_mine ? (int64_t)((ss_item / ROWS) * ss_per + ss_q * ss_cnt) * a.ss_ld + col0 +
                                           ss_item % ROWS
                                     : 0);
#pragma unroll
    for (int t = 0; t < SSMAX; ++t) ssv[t] = p[(int64_t)min(t, ss_cnt - 1) * a.ss_ld];
  }
  auto ss_store = [&]() {  // norm_part[q][grp][row]
    if (ss_early && ss_q < nq) {
      float s = 0.f;
      asm volatile("" : "+v"(s));  // the sum starts here, not next to the loads (no early wait)
      if (ss_mine)
#pragma unroll
        for (int t = 0; t < SSMAX; ++t)
          if (t < ss_cnt) s += ssv[t];
      norm_part[(ss_q * 16 + ss_item / ROWS) * ROWS + ss_item % ROWS] = s;
    }
  };
  // ... and the residual rows this wave's epilogue adds to
  float4 hres[RT][NB];
  if constexpr (EPI == EPI_RESIDUAL) {
    if (wave == 0) {
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int i = 0; i < RT; ++i)
          if (8 * c + (lane & 7) < rows_valid)
            hres[i][c] = *reinterpret_cast<const float4*>(a.out + (int64_t)(col0 + 8 * c + (lane & 7)) * a.ldo +
                                                          sub_row[i] + 4 * (lane >> 4));
    }
  }

  bool valu_done = false;
  if constexpr (FMT == FMT_BF16 && NB == 1 && VALU_ROWS > 0) {
    // Vector-ALU inner products (a build option kept for comparison with the matrix cores at
    // B <= VALU_ROWS). Lane l holds inputs 8g..8g+7 (g = l/16) of row l%16 of each 32-input chunk;
    // the activations it needs are columns b (hi) and 8 + b (lo) of the fragment's lanes 16g + b and
    // 16g + 8 + b. Every lane keeps RT x VALU_ROWS partial sums; a VALU_DEPTH-chunk ring of loads.
    const int chunks = kw / 32;
    if (rows_valid <= VALU_ROWS && chunks % VALU_DEPTH == 0) {
      constexpr int BV = VALU_ROWS > 0 ? VALU_ROWS : 1;  // (array extents of the default build)
      const uint16_t* xg = xr[0] - 8 * lane + 128 * (lane >> 4);
      struct VBuf {
        u32x4_t A[RT];
        u32x4_t H[BV], L[BV];
      };
      auto vload = [&](VBuf& f, int ch) {
#pragma unroll
        for (int i = 0; i < RT; ++i)
          f.A[i] = load_stream(reinterpret_cast<const uint16_t*>(wr[i]) + (int64_t)ch * 512);
#pragma unroll
        for (int b = 0; b < BV; ++b) {
          f.H[b] = *reinterpret_cast<const u32x4_t*>(xg + ch * 512 + 8 * b);
          f.L[b] = *reinterpret_cast<const u32x4_t*>(xg + ch * 512 + 8 * (8 + b));
        }
      };
      float pv[RT][BV];
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int b = 0; b < BV; ++b) pv[i][b] = 0.f;
      auto vcompute = [&](const VBuf& f) {
        float xv[BV][8];
#pragma unroll
        for (int b = 0; b < BV; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {  // word q: input 2q in the low half, 2q + 1 in the high half
            xv[b][2 * q] = __uint_as_float(f.H[b][q] << 16) + __uint_as_float(f.L[b][q] << 16);
            xv[b][2 * q + 1] = __uint_as_float(f.H[b][q] & 0xFFFF0000u) + __uint_as_float(f.L[b][q] & 0xFFFF0000u);
          }
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float w0 = __uint_as_float(f.A[i][q] << 16), w1 = __uint_as_float(f.A[i][q] & 0xFFFF0000u);
#pragma unroll
            for (int b = 0; b < BV; ++b) pv[i][b] = fmaf(w1, xv[b][2 * q + 1], fmaf(w0, xv[b][2 * q], pv[i][b]));
          }
      };
      VBuf vb[VALU_DEPTH];
#pragma unroll
      for (int j = 0; j < VALU_DEPTH; ++j) {
        vload(vb[j], j);
        __builtin_amdgcn_sched_barrier(0);
      }
      ss_store();
      int ch = 0;
      for (; ch + VALU_DEPTH < chunks; ch += VALU_DEPTH) {
#pragma unroll
        for (int j = 0; j < VALU_DEPTH; ++j) {
          vcompute(vb[j]);
          __builtin_amdgcn_sched_barrier(0);
          vload(vb[j], ch + VALU_DEPTH + j);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int j = 0; j < VALU_DEPTH; ++j) vcompute(vb[j]);
      // sums over the 4 input groups, then into the matrix-core accumulator layout: lane l holds
      // rows 4g + e of column l%16; columns b < BV (hi) take the whole product, all others zero
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int b = 0; b < BV; ++b) {
          pv[i][b] += __shfl_xor(pv[i][b], 16, 64);
          pv[i][b] += __shfl_xor(pv[i][b], 32, 64);
        }
      const int col = lane & 15;
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = 0.f;
#pragma unroll
          for (int b = 0; b < BV; ++b) {
            const float t = __shfl(pv[i][b], 4 * (lane >> 4) + e, 64);
            if (col == b) v = t;
          }
          acc[i][0][e] = v;
        }
      valu_done = true;
    }
  }

  if constexpr (FMT == FMT_BF16) {
   if (!valu_done) {
    struct Buf {
      u32x4_t A[UC][RT];
      bf16x8_t X[UC][NB];
    };
    auto load = [&](Buf& f, int st) {
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int i = 0; i < RT; ++i)
          f.A[u][i] = load_stream(reinterpret_cast<const uint16_t*>(wr[i]) + (int64_t)(st * UC + u) * 512);
      // padding rows of a fragment share its cache lines with the valid rows and feed only padding
      // outputs: they are loaded like the rest (no branch, so load completion counts stay static)
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int c = 0; c < NB; ++c) f.X[u][c] = load_frag(xr[c] + (st * UC + u) * 512);
    };
    auto compute = [&](const Buf& f) {
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int c = 0; c < NB; ++c) acc[i][c] = mfma(as_frag(f.A[u][i]), f.X[u][c], acc[i][c]);
    };
    // Every load in the prologue and the steady-state loop is unconditional, so the compiler's
    // load-completion waits stay exact (wait for one buffer while the other is in flight); the
    // last 2 or 3 stages are peeled. The plan guarantees total >= 2.
    // Scheduling barriers keep each buffer's loads together and in program order, so waiting for
    // one buffer never waits for the other's.
    const int total = kw / (32 * UC);
    Buf b0, b1;
    load(b0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load(b1, 1);
    __builtin_amdgcn_sched_barrier(0);
    ss_store();  // waits for the sums only: they were requested before the weights
    int st = 0;
    for (; st + 3 < total; st += 2) {
      compute(b0);
      __builtin_amdgcn_sched_barrier(0);
      load(b0, st + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(b1);
      __builtin_amdgcn_sched_barrier(0);
      load(b1, st + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    compute(b0);
    if (st + 2 < total) {
      __builtin_amdgcn_sched_barrier(0);
      load(b0, st + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(b1);
      compute(b0);
    } else {
      compute(b1);
    }
   }
  } else {
    // int4: 128 inputs per stage; the same two-buffer pipeline as the bf16 path
    const Int4Consts kc = Int4Consts::make();
    const ScaleRows<RT> srows = scale_rows<RT>(a, sub_row, lane >> 4);
    struct QBuf {
      u32x4_t Wq[RT];
      uint4 SB[RT][2];
      bf16x8_t X[4][NB];
    };
    auto qload = [&](QBuf& f, int st) {
#pragma unroll
      for (int i = 0; i < RT; ++i) f.Wq[i] = load_stream(reinterpret_cast<const uint32_t*>(wr[i]) + (int64_t)st * 256);
      load_scales<RT>(srows, k0 + st * 128, f.SB);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < NB; ++c) f.X[j][c] = load_frag(xr[c] + (4 * st + j) * 512);
    };
    const int total = kw / 128;  // >= 2 (plan)
    QBuf b0, b1;
    qload(b0, 0);
    __builtin_amdgcn_sched_barrier(0);
    qload(b1, 1);
    __builtin_amdgcn_sched_barrier(0);
    ss_store();
    int st = 0;
    for (; st + 3 < total; st += 2) {
      int4_block<RT, NB>(acc, b0.Wq, b0.SB, b0.X, kc);
      __builtin_amdgcn_sched_barrier(0);
      qload(b0, st + 2);
      __builtin_amdgcn_sched_barrier(0);
      int4_block<RT, NB>(acc, b1.Wq, b1.SB, b1.X, kc);
      __builtin_amdgcn_sched_barrier(0);
      qload(b1, st + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    int4_block<RT, NB>(acc, b0.Wq, b0.SB, b0.X, kc);
    if (st + 2 < total) {
      __builtin_amdgcn_sched_barrier(0);
      qload(b0, st + 2);
      __builtin_amdgcn_sched_barrier(0);
      int4_block<RT, NB>(acc, b1.Wq, b1.SB, b1.X, kc);
      int4_block<RT, NB>(acc, b0.Wq, b0.SB, b0.X, kc);
    } else {
      int4_block<RT, NB>(acc, b1.Wq, b1.SB, b1.X, kc);
    }
  }

  // fixed-order reduction of the K slices through LDS; the norm partials are gathered meanwhile
  if (wave > 0) {
    float* dst = red + (size_t)(wave - 1) * NACC * 64;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[((i * NB + c) * 4 + e) * 64 + lane] = acc[i][c][e];
  }
  if (a.ss && !ss_early) norm_partials<ROWS>(a, col0, rows_valid, norm_part);
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < nw; ++w) {
    const float* src = red + (size_t)(w - 1) * NACC * 64;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][c][e] += src[((i * NB + c) * 4 + e) * 64 + lane];
  }
  if (ns > 1) {
    // K split over workgroups (to even out the work per compute unit): wave 0 of each stores its
    // sums (agent scope); the last to arrive adds the splits in order
    constexpr int TILE_F = NACC * 64;
    const int64_t base = (int64_t)(tile - split_from) * splits * TILE_F;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c)
        store_agent_x4(a.part, (int)((base + (int64_t)split * TILE_F + ((i * NB + c) * 64 + lane) * 4) * 4), acc[i][c]);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the partial stores are done
    int last = 0;
    if (lane == 0)
      last = __hip_atomic_fetch_add(a.counters + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == splits - 1;
    if (!__shfl(last, 0, 64)) return;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c) acc[i][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // several splits' loads in flight (one memory latency per MB splits), added in split order
    constexpr int MB = RT * NB <= 4 ? 4 : (RT * NB <= 8 ? 2 : 1);
    for (int sp0 = 0; sp0 < splits; sp0 += MB) {
      f32x4_t t[MB][RT][NB];
#pragma unroll
      for (int u = 0; u < MB; ++u)
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int c = 0; c < NB; ++c)
            t[u][i][c] = load_agent_x4(
                a.part, (int)((base + (int64_t)min(sp0 + u, splits - 1) * TILE_F + ((i * NB + c) * 64 + lane) * 4) * 4));
#pragma unroll
      for (int u = 0; u < MB; ++u)
        if (sp0 + u < splits)
#pragma unroll
          for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int c = 0; c < NB; ++c) acc[i][c] += t[u][i][c];
    }
    if (lane == 0) __hip_atomic_store(a.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  float inv[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c)
    inv[c] = a.ss ? norm_inv<ROWS>(a, norm_part, 8 * c + (lane & 7), ss_early ? nq : 1) : 1.f;
  epilogue<RT, NB, EPI>(a, acc, sub_row, col0, rows_valid, inv, lane, EPI == EPI_RESIDUAL ? &hres : nullptr);
}

// ============================================================================ row split

template <int RT, int NB, int EPI, int FMT, int UC>
__global__ __launch_bounds__(256) void rowsplit_gemm_kernel(SkinnyArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int ROWS = 8 * NB;  // activation rows: NB groups of 8
  constexpr int NACC = RT * NB * 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int blk = blockIdx.x, split = blockIdx.y, S = gridDim.y, xblk = blockIdx.z;
  const int K = a.K, Kr = K / S, kbeg = split * Kr, KC = a.kc;
  const int col0 = xblk * ROWS;
  const int rows_valid = min(ROWS, a.rows - col0);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);  // [NB][KC/32] fragments of 512 elements
  float* norm_part = reinterpret_cast<float*>(smem + (size_t)NB * KC * 32);  // [16][ROWS]
  __shared__ int s_last;

  // workgroup tile = 4 waves x RT subtiles (SwiGLU: 64 features, gate and up rows per wave)
  int sub_row[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) sub_row[i] = subtile_row<RT, EPI>(a, blk * 4 + wave, i);
  const void* wr[RT];
  weight_ptrs<RT, FMT>(a, sub_row, K, kbeg, lane, wr);

  f32x4_t acc[RT][NB];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[i][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // stage activation chunk [kc0, kc0 + KC): whole fragments of the valid 8-row groups
  const int kfc = KC >> 5;
  const int valid_groups = (rows_valid + 7) >> 3;
  auto stage_x = [&](int kc0) {
    __syncthreads();  // the previous chunk has been consumed
    const int per_group = kfc * 64;  // 16-byte words of one group's chunk
    for (int idx = threadIdx.x; idx < valid_groups * per_group; idx += 256) {
      const int c = idx / per_group, w = idx - c * per_group;
      if (8 * c + (w & 7) >= rows_valid) continue;  // word w holds row w%8 of its fragment
      const uint16_t* src = a.x + ((int64_t)((col0 >> 3) + c) * (K >> 5) + (kc0 >> 5)) * 512 + 8 * w;
      *reinterpret_cast<uint4*>(xs + (c * kfc) * 512 + 8 * w) = *reinterpret_cast<const uint4*>(src);
    }
    __syncthreads();
  };
  auto xlds = [&](int c, int kf) { return load_frag(xs + (c * kfc + kf) * 512 + 8 * lane); };

  if constexpr (FMT == FMT_BF16) {
    const int spc = KC / (32 * UC), total = Kr / (32 * UC);
    u32x4_t A0[UC][RT], A1[UC][RT];
    auto loadw = [&](u32x4_t (&A)[UC][RT], int st) {
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int i = 0; i < RT; ++i)
          A[u][i] = load_stream(reinterpret_cast<const uint16_t*>(wr[i]) + (int64_t)(st * UC + u) * 512);
    };
    auto compute = [&](const u32x4_t (&A)[UC][RT], int st) {
      const int kf0 = (st % spc) * UC;
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          const bf16x8_t x = xlds(c, kf0 + u);
#pragma unroll
          for (int i = 0; i < RT; ++i) acc[i][c] = mfma(as_frag(A[u][i]), x, acc[i][c]);
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
    const int spc = KC / 128, total = Kr / 128;
    const Int4Consts kc = Int4Consts::make();
    const ScaleRows<RT> srows = scale_rows<RT>(a, sub_row, lane >> 4);
    for (int st = 0; st < total; ++st) {
      if (st % spc == 0) stage_x(kbeg + (st / spc) * KC);
      u32x4_t Wq[RT];
      uint4 SB[RT][2];
      bf16x8_t X[4][NB];
#pragma unroll
      for (int i = 0; i < RT; ++i) Wq[i] = load_stream(reinterpret_cast<const uint32_t*>(wr[i]) + (int64_t)st * 256);
      load_scales<RT>(srows, kbeg + st * 128, SB);
      const int kf0 = (st % spc) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < NB; ++c) X[j][c] = xlds(c, kf0 + j);
      int4_block<RT, NB>(acc, Wq, SB, X, kc);
    }
  }

  // split over workgroups: partial tiles to the workspace; the last workgroup of the row block adds
  // them. Partials and the arrival counter use agent-scope atomic accesses (coherent across the XCDs'
  // L2 caches); each wave waits for its stores to be acknowledged (vmcnt 0) before arrival is counted,
  // which avoids the full L2 write-back and invalidate of a device-wide fence.
  if (S > 1) {
    // partial tile of (split, wave): [i][c][lane] f32x4, 16 bytes per lane and subtile
    const int64_t base = (int64_t)blk * S * 4 * NACC * 64;
    const int64_t mine = base + ((int64_t)split * 4 + wave) * NACC * 64;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c)
        store_agent_x4(a.part, (int)((mine + ((i * NB + c) * 64 + lane) * 4) * 4), acc[i][c]);
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
      const int64_t src = base + ((int64_t)s * 4 + wave) * NACC * 64;
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int c = 0; c < NB; ++c)
          acc[i][c] += load_agent_x4(a.part, (int)((src + ((i * NB + c) * 64 + lane) * 4) * 4));
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.counters + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  float inv[NB];
  if (a.ss) {
    norm_partials<ROWS>(a, col0, rows_valid, norm_part);
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < NB; ++c) inv[c] = a.ss ? norm_inv<ROWS>(a, norm_part, 8 * c + (lane & 7), 1) : 1.f;
  epilogue<RT, NB, EPI>(a, acc, sub_row, col0, rows_valid, inv, lane, nullptr);
}

// ============================================================================ dense tiles

// Many activation rows: WN x WM waves of 64 weight rows x 8*NBW activation rows each, so a
// workgroup covers TN = 64 WN weight rows x TM = 8 NBW WM activation rows (prefill: 256 x 128 with
// 64 x 64 waves; decode steps: 128 x 64 or 128 x 32 with 64 x 32 waves). Each stage copies one
// 32-input fragment column to LDS (the fragments are already MFMA operands), double-buffered with
// one barrier per stage and two stages of loads in flight: both operands for tiles of 4 activation
// groups per wave, the activations only for tiles of 8 (their weight operands go straight to
// registers). SwiGLU tiles hold TN/2 gate rows and the matching up rows. bf16 weights only. With
// splits > 1 (one row tile), workgroup (tile, s) adds the inputs [s K/splits, (s + 1) K/splits);
// the last workgroup of a tile to arrive adds the partial tiles in order (agent-scope 16-byte
// accesses and an arrival counter, as the row split).
#ifndef CBD_DENSE_DEPTH
#define CBD_DENSE_DEPTH 2
#endif

namespace {
// LDS of a dense workgroup: two stages of (4 wn + nbw wm) fragments, 1/rms per activation row
inline size_t dense_lds(int wn, int wm, int nbw) {
  return (size_t)2 * (4 * wn + nbw * wm) * 512 * 2 + 8 * nbw * wm * 4;
}

// weight row of subtile f (0 .. NWF-1) of the workgroup's tile
template <int EPI, int NWF>
CBD_DEVICE int dense_row(const SkinnyArgs& a, int n0, int f) {
  if constexpr (EPI == EPI_SWIGLU)
    return f < NWF / 2 ? n0 + 16 * f : a.seg_end[0] + n0 + 16 * (f - NWF / 2);
  return n0 + 16 * f;
}
}  // namespace

template <int EPI, int WN, int WM, int NBW>
__global__ __launch_bounds__(64 * WN * WM, 2) void dense_gemm_kernel(SkinnyArgs a, int tiles_n, int splits) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int RT = 4, NB = NBW;          // a wave: 4 weight subtiles x NBW activation groups
  static_assert(NBW % 4 == 0, "activation groups come 4 at a time");
  constexpr int D = CBD_DENSE_DEPTH;       // register stages in flight (even)
  constexpr int NW = WN * WM, NTH = 64 * NW;
  constexpr int TN = 64 * WN, TM = 8 * NBW * WM;  // weight rows and activation rows of the tile
  constexpr int NWF = 4 * WN, FR = NWF + NBW * WM;  // fragments per stage: weight subtiles, then groups
  constexpr int PER = FR / NW;             // fragment copies per thread and stage
  static_assert(FR % NW == 0, "fragments per stage split evenly over the waves");
  constexpr int STAGE = FR * 512;          // elements of one LDS stage
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);  // 2 stages
  float* inv_s = reinterpret_cast<float*>(smem + 2 * STAGE * 2);  // [TM]
  __shared__ int s_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wn = wave % WN, wm = wave / WN;
  const int tiles_m = (a.rows + TM - 1) / TM;
  int tn, tm, split = 0;
  if (splits == 1) {
    // XCD-aware tile order: workgroups go to the 8 XCDs round-robin, so the ones an XCD runs together
    // (ids x, x + 8, x + 16, ...) get one 8 x 8 block of tiles and reuse its weight and activation
    // fragments from that XCD's L2. Ids that fall outside the tile grid return.
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int super = (j >> 6) * 8 + xcd, r = j & 63;
    const int super_n = (tiles_n + 7) >> 3;
    tn = (super % super_n) * 8 + (r & 7);
    tm = (super / super_n) * 8 + (r >> 3);
    if (tn >= tiles_n || tm >= tiles_m) return;
  } else {
    tn = blockIdx.x / splits;
    split = blockIdx.x - tn * splits;
    tm = 0;
  }
  const int n0 = tn * (EPI == EPI_SWIGLU ? TN / 2 : TN);
  const int m0 = tm * TM;
  const int K = a.K, nk_all = K >> 5, nk = nk_all / splits, kf0 = split * nk;

  // this thread's fragment copies per stage: f = wave + NW i (weights first, then activation groups)
  const uint16_t* src[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = wave + NW * i;
    if (f < NWF) {
      const int grow = dense_row<EPI, NWF>(a, n0, f);
      const int sg = seg_of(a, grow);
      const int tr = (grow - seg_begin(a, sg)) >> 4;
      src[i] = reinterpret_cast<const uint16_t*>(a.w[sg]) + ((int64_t)tr * nk_all + kf0) * 512 + 8 * lane;
    } else {
      src[i] = a.x + ((int64_t)((m0 >> 3) + (f - NWF)) * nk_all + kf0) * 512 + 8 * lane;
    }
  }
  // global -> registers -> LDS; D register sets keep the loads of the next D stages in flight
  auto fetch = [&](u32x4_t (&r)[PER], int kf) {  // cached loads: other tiles reuse them
#pragma unroll
    for (int i = 0; i < PER; ++i) r[i] = *reinterpret_cast<const u32x4_t*>(src[i] + (int64_t)kf * 512);
  };
  auto put = [&](const u32x4_t (&r)[PER], int buf) {  // a fragment is a 1 KB copy
#pragma unroll
    for (int i = 0; i < PER; ++i)
      *reinterpret_cast<u32x4_t*>(lds + buf * STAGE + (wave + NW * i) * 512 + 8 * lane) = r[i];
  };
  u32x4_t rr[D][PER];
  auto prologue = [&]() {
    fetch(rr[0], 0);
    put(rr[0], 0);
    __syncthreads();
    // stages past the last refetch the last one (unused): loads stay unconditional
    // (scheduling barriers keep the loads in register-set order here and in the loop, so that the
    // waits at the loop head count the same outstanding loads on entry and on the back edge)
#pragma unroll
    for (int j = 0; j < D; ++j) {
      fetch(rr[j], min(1 + j, nk - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x4_t acc[RT][NB];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[i][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // LDS fragments of this wave: weights (4 subtiles; SwiGLU: 2 gate, then their 2 up), activations
  int fa[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    if constexpr (EPI == EPI_SWIGLU) fa[i] = i < 2 ? 2 * wn + i : NWF / 2 + 2 * wn + (i - 2);
    else fa[i] = 4 * wn + i;
  }
  auto compute = [&](int buf) {  // activation groups 4 at a time (registers)
    const uint16_t* st = lds + buf * STAGE;
    bf16x8_t A[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) A[i] = *reinterpret_cast<const bf16x8_t*>(st + fa[i] * 512 + 8 * lane);
#pragma unroll
    for (int c0 = 0; c0 < NB; c0 += 4) {
      bf16x8_t X[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        X[c] = *reinterpret_cast<const bf16x8_t*>(st + (NWF + NBW * wm + c0 + c) * 512 + 8 * lane);
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c0 + c] = mfma(A[i], X[c], acc[i][c0 + c]);
    }
  };
  if constexpr (NBW == 8) {
    // Tiles of 8 activation groups per wave (prefill; 64-row decode lm_head): the weight operands
    // are loaded straight into registers (a ring of two stages: the set a stage used is refilled
    // with the stage after next once its products are issued), and the LDS stages hold the
    // activation fragments only, double-buffered. The two waves sharing weight rows load the same
    // fragments (the second from L2). The activations of the next stage are read from LDS while the
    // matrix cores still work on this one, so a stage starts with its first operands in registers.
    // Stage s: first half (groups 0..3, group by group; each freed X register receives group 4 + c
    // of the stage); put stage s + 1 into the other buffer and synchronise (every wave is then done
    // with that buffer's previous contents: their reads completed before the last barrier); second
    // half (groups 4..7): groups 4 and 5 first, their registers receiving groups 0 and 1 of stage
    // s + 1; then groups 6 and 7, after which their registers receive groups 2 and 3 of stage s + 1.
    // Measured against staging the weights through LDS as well (prefill gate/up at 7797 tokens):
    // 3303 -> 3203 us with the read-ahead, 3222 us for neither.
    constexpr int FX = NBW * WM, PX = FX / NW;  // activation fragments per stage, copies per thread
    static_assert(FX % NW == 0, "activation fragments split evenly over the waves");
    constexpr int SX = FX * 512;
    const uint16_t* xsrc[PX];
#pragma unroll
    for (int p = 0; p < PX; ++p)
      xsrc[p] = a.x + ((int64_t)((m0 >> 3) + wave + NW * p) * nk_all + kf0) * 512 + 8 * lane;
    const uint16_t* wsrc[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int grow = dense_row<EPI, NWF>(a, n0, fa[i]);
      const int sg = seg_of(a, grow);
      wsrc[i] = reinterpret_cast<const uint16_t*>(a.w[sg]) +
                ((int64_t)((grow - seg_begin(a, sg)) >> 4) * nk_all + kf0) * 512 + 8 * lane;
    }
    auto xfetch = [&](u32x4_t (&r)[PX], int kf) {
#pragma unroll
      for (int p = 0; p < PX; ++p) r[p] = *reinterpret_cast<const u32x4_t*>(xsrc[p] + (int64_t)kf * 512);
    };
    auto xput = [&](const u32x4_t (&r)[PX], int buf) {
#pragma unroll
      for (int p = 0; p < PX; ++p)
        *reinterpret_cast<u32x4_t*>(lds + buf * SX + (wave + NW * p) * 512 + 8 * lane) = r[p];
    };
    auto wfetch = [&](u32x4_t (&w)[RT], int kf) {  // cached loads: the other activation tiles reuse them
#pragma unroll
      for (int i = 0; i < RT; ++i) w[i] = *reinterpret_cast<const u32x4_t*>(wsrc[i] + (int64_t)kf * 512);
    };
    const uint16_t* xw = lds + (NBW * wm) * 512 + 8 * lane;
    auto rdX = [&](int buf, int c) { return *reinterpret_cast<const bf16x8_t*>(xw + buf * SX + c * 512); };
    u32x4_t xr[D][PX], W[2][RT];
    xfetch(xr[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    wfetch(W[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    wfetch(W[1], min(1, nk - 1));
    __builtin_amdgcn_sched_barrier(0);
    xput(xr[0], 0);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < D; ++j) {
      xfetch(xr[j], min(1 + j, nk - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8_t X[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) X[c] = rdX(0, c);
    for (int kf = 0; kf < nk; kf += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {  // stage s = kf + j: activations in buffer s & 1, weights in W[s & 1]
        const int buf = j & 1, nbuf = buf ^ 1;
        u32x4_t (&A)[RT] = W[j & 1];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int i = 0; i < RT; ++i) acc[i][c] = mfma(as_frag(A[i]), X[c], acc[i][c]);
          X[c] = rdX(buf, 4 + c);
          __builtin_amdgcn_sched_barrier(0);
        }
        xput(xr[j], nbuf);
        __syncthreads();
        xfetch(xr[j], min(kf + j + 1 + D, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int i = 0; i < RT; ++i) acc[i][4 + c] = mfma(as_frag(A[i]), X[c], acc[i][4 + c]);
          X[c] = rdX(nbuf, c);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < RT; ++i) {
          acc[i][6] = mfma(as_frag(A[i]), X[2], acc[i][6]);
          acc[i][7] = mfma(as_frag(A[i]), X[3], acc[i][7]);
        }
        __builtin_amdgcn_sched_barrier(0);
        X[2] = rdX(nbuf, 2);
        X[3] = rdX(nbuf, 3);
        wfetch(A, min(kf + j + 2, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
  prologue();
  // stage s is in LDS buffer s & 1; register set s % D holds stage s + 1 and is put after computing
  // s, then refilled with stage s + 1 + D. nk is a multiple of D (and even), so the loop body has no
  // branch and the load waits stay exact.
  for (int kf = 0; kf < nk; kf += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      compute(j & 1);
      put(rr[j], (j + 1) & 1);
      __syncthreads();
      fetch(rr[j], min(kf + j + 1 + D, nk - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  }

  if (splits > 1) {
    // partial tile of (tile, split, wave): hi and lo products added first, then [i][c][32 lanes]
    // f32x4 from the lanes that hold a low half (16 bytes per lane and subtile); the merged sums go
    // back to those lanes, zero to the others, so the epilogue's hi + lo addition leaves them as is
    constexpr int TILE_F = NW * RT * NB * 32 * 4;  // floats of one workgroup's partial
    const int64_t base = (int64_t)tn * splits * TILE_F;
    const int l32 = ((lane >> 4) << 3) | (lane & 7);
    const bool holder = (lane & 8) == 0;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        f32x4_t v = acc[i][c];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += __shfl_xor(v[e], 8, 64);
        if (holder)
          store_agent_x4(a.part, (int)((base + (int64_t)split * TILE_F + ((wave * RT + i) * NB + c) * 128 + l32 * 4) * 4),
                         v);
      }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are done
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(a.counters + tn, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == splits - 1;
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c) acc[i][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int MB = NB <= 4 ? 2 : 1;  // splits whose loads are in flight together (registers)
    if (holder)  // added in split order
      for (int sp0 = 0; sp0 < splits; sp0 += MB) {
        f32x4_t t[MB][RT][NB];
#pragma unroll
        for (int u = 0; u < MB; ++u)
#pragma unroll
          for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int c = 0; c < NB; ++c)
              t[u][i][c] = load_agent_x4(a.part, (int)((base + (int64_t)min(sp0 + u, splits - 1) * TILE_F +
                                                        ((wave * RT + i) * NB + c) * 128 + l32 * 4) * 4));
#pragma unroll
        for (int u = 0; u < MB; ++u)
          if (sp0 + u < splits)
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
              for (int c = 0; c < NB; ++c) acc[i][c] += t[u][i][c];
      }
    if (tid == 0) __hip_atomic_store(a.counters + tn, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // 1/rms of the tile's rows, added in the same fixed order as the other kernels (per group of 16
  // partials in order, then the 16 groups in order). Computed after the product, by the workgroups
  // that run the epilogue only, with each thread's loads for 8 partials of its 4 items in flight
  // together; the stage buffers hold the per-group sums.
  if (a.ss) {
    constexpr int IPT = 16 * TM / NTH;  // (row, group) items per thread
    static_assert(16 * TM % NTH == 0, "items split evenly");
    __syncthreads();  // every wave is past its last read of the stage buffers
    float* part = reinterpret_cast<float*>(lds);  // [16][TM]
    const int per = a.ss_tiles / 16;
    const float* q[IPT];
    float sum[IPT];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int i = tid + NTH * j, r = i % TM, grp = i / TM;
      q[j] = a.ss + (int64_t)grp * per * a.ss_ld + min(m0 + r, a.rows - 1);  // rows past the last: unused
      sum[j] = 0.f;
    }
    for (int t0 = 0; t0 < per; t0 += 8) {
      float v[IPT][8];
#pragma unroll
      for (int j = 0; j < IPT; ++j)
#pragma unroll
        for (int u = 0; u < 8; ++u) v[j][u] = q[j][(int64_t)min(t0 + u, per - 1) * a.ss_ld];
#pragma unroll
      for (int j = 0; j < IPT; ++j)
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (t0 + u < per) sum[j] += v[j][u];
    }
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int i = tid + NTH * j;
      part[(i / TM) * TM + i % TM] = sum[j];
    }
    __syncthreads();
    if (tid < TM) {
      float s2 = 0.f;
      for (int grp = 0; grp < 16; ++grp) s2 += part[grp * TM + tid];
      inv_s[tid] = 1.0f / sqrtf(s2 / a.norm_dim + a.eps);
    }
    __syncthreads();
  }

  int sub_row[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) sub_row[i] = dense_row<EPI, NWF>(a, n0, fa[i]);
  const int col0 = m0 + 8 * NBW * wm;
  const int rows_valid = min(8 * NBW, a.rows - col0);
  if (rows_valid <= 0) return;
  // the epilogue takes the activation groups 4 at a time (registers)
#pragma unroll
  for (int c0 = 0; c0 < NB; c0 += 4) {
    f32x4_t part[RT][4];
    float inv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      inv[c] = a.ss ? inv_s[8 * NBW * wm + 8 * (c0 + c) + (lane & 7)] : 1.f;
#pragma unroll
      for (int i = 0; i < RT; ++i) part[i][c] = acc[i][c0 + c];
    }
    epilogue<RT, 4, EPI>(a, part, sub_row, col0 + 8 * c0, rows_valid - 8 * c0, inv, lane, nullptr);
  }
}

// ============================================================================ wide k split

// 9..64 activation rows (decode steps of wide batches): a workgroup of 4 waves takes one tile of
// 64 weight rows (4 subtiles; SwiGLU: 32 gate rows and the 32 up rows of the same features) over one
// of `splits` K ranges; each wave streams a contiguous quarter of that range with all NB activation
// groups, so every activation fragment read from L2 feeds 4 weight fragments (the k-split kernel
// feeds one). The waves' sums are added through LDS in wave order; wave w then owns the groups
// c = w (mod 4): with splits > 1 it stores their partial tiles (agent scope) and the last workgroup
// of a tile to arrive adds the splits in order, computes 1/rms of the rows if the input is normed,
// and runs the epilogue of the groups its waves own.
namespace {
constexpr int kWideWaves = 4;
inline size_t wide_lds(int nb, int rt) { return (size_t)kWideWaves * nb * rt * 32 * 16 + 16 * 8 * nb * 4 + 8 * nb * 4; }
}  // namespace

template <int EPI, int NB, int UC, int RT>
__global__ __launch_bounds__(64 * kWideWaves, (NB == 8 && RT == 4) ? 1 : 2) void wide_ksplit_kernel(SkinnyArgs a, int splits) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int NW = kWideWaves, NTH = 64 * NW, ROWS = 8 * NB;
  f32x4_t* red = reinterpret_cast<f32x4_t*>(smem);                          // [NW][NB][RT][32]
  float* npart = reinterpret_cast<float*>(smem + NW * NB * RT * 32 * 16);  // [16][ROWS]
  float* inv_s = npart + 16 * ROWS;                                        // [ROWS]
  __shared__ int s_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tile = blockIdx.x / splits, split = blockIdx.x - tile * splits;
  const int K = a.K, kr = K / splits, kw = kr / NW, k0 = split * kr + wave * kw;

  int sub_row[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) sub_row[i] = subtile_row<RT, EPI>(a, tile, i);
  const void* wr[RT];
  weight_ptrs<RT, FMT_BF16>(a, sub_row, K, k0, lane, wr);
  const uint16_t* xr = a.x + (int64_t)(k0 >> 5) * 512 + 8 * lane;  // group c at + c (K/32) 512
  const int64_t xg = (int64_t)(K >> 5) * 512;

  f32x4_t acc[RT][NB];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[i][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Buf {
    u32x4_t A[UC][RT];
    bf16x8_t X[UC][NB];
  };
  auto load = [&](Buf& f, int st) {
#pragma unroll
    for (int u = 0; u < UC; ++u)
#pragma unroll
      for (int i = 0; i < RT; ++i)
        f.A[u][i] = load_stream(reinterpret_cast<const uint16_t*>(wr[i]) + (int64_t)(st * UC + u) * 512);
    // padding rows of the last groups are loaded like the rest (the workspace holds whole groups)
#pragma unroll
    for (int u = 0; u < UC; ++u)
#pragma unroll
      for (int c = 0; c < NB; ++c) f.X[u][c] = load_frag(xr + c * xg + (st * UC + u) * 512);
  };
  auto compute = [&](const Buf& f) {
#pragma unroll
    for (int u = 0; u < UC; ++u)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int i = 0; i < RT; ++i) acc[i][c] = mfma(as_frag(f.A[u][i]), f.X[u][c], acc[i][c]);
  };
  // the k-split kernel's two-buffer pipeline: unconditional loads, each buffer's loads kept together
  // by scheduling barriers, the last 2 or 3 stages peeled (the plan guarantees total >= 2)
  const int total = kw / (32 * UC);
  Buf b0, b1;
  load(b0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(b1, 1);
  __builtin_amdgcn_sched_barrier(0);
  int st = 0;
  for (; st + 3 < total; st += 2) {
    compute(b0);
    __builtin_amdgcn_sched_barrier(0);
    load(b0, st + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(b1);
    __builtin_amdgcn_sched_barrier(0);
    load(b1, st + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  compute(b0);
  if (st + 2 < total) {
    __builtin_amdgcn_sched_barrier(0);
    load(b0, st + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(b1);
    compute(b0);
  } else {
    compute(b1);
  }

  // hi + lo, then the waves' sums through LDS: lanes with l & 8 clear hold (row l%8, outputs 4 g..)
  const int l32 = ((lane >> 4) << 3) | (lane & 7);
  const bool holder = (lane & 8) == 0;
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int c = 0; c < NB; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][c][e] += __shfl_xor(acc[i][c][e], 8, 64);
      if (holder) red[((wave * NB + c) * RT + i) * 32 + l32] = acc[i][c];
    }
  __syncthreads();
  // wave w adds the groups c = w (mod NW) over the waves in order; the sums go to the holder lanes,
  // zero to the others (the epilogue's hi + lo addition then leaves them as they are)
#pragma unroll
  for (int c = 0; c < NB; ++c)
    if (c % NW == wave) {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        f32x4_t v = red[(c * RT + i) * 32 + l32];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[((w * NB + c) * RT + i) * 32 + l32];
        acc[i][c] = holder ? v : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }

  // the residual rows this wave's epilogue adds to (groups c = wave + NW q), requested before the
  // merge and the norm so that their latency overlaps them
  constexpr int NQ = NB / NW > 0 ? NB / NW : 1;
  float4 hpre[NQ][RT][1];
  auto prefetch_h = [&]() {
    if constexpr (EPI == EPI_RESIDUAL) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int row = 8 * (wave + NW * q) + (lane & 7);
        if (wave + NW * q < NB && row < a.rows && holder)
#pragma unroll
          for (int i = 0; i < RT; ++i)
            hpre[q][i][0] = *reinterpret_cast<const float4*>(a.out + (int64_t)row * a.ldo + sub_row[i] + 4 * (lane >> 4));
      }
    }
  };

  if (splits > 1) {
    constexpr int TILE_F = NB * RT * 32 * 4;  // floats of one workgroup's partial tile
    const int64_t base = (int64_t)tile * splits * TILE_F;
#pragma unroll
    for (int c = 0; c < NB; ++c)
      if (c % NW == wave && holder)
#pragma unroll
        for (int i = 0; i < RT; ++i)
          store_agent_x4(a.part, (int)((base + (int64_t)split * TILE_F + ((c * RT + i) * 32 + l32) * 4) * 4), acc[i][c]);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are done
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(a.counters + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == splits - 1;
    __syncthreads();
    if (!s_last) return;
    prefetch_h();
    // the splits' partial tiles with up to 4 splits' loads in flight (one memory latency per 4
    // splits), added in split order
#pragma unroll
    for (int c = 0; c < NB; ++c)
      if (c % NW == wave) {
#pragma unroll
        for (int i = 0; i < RT; ++i) acc[i][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (holder)
          for (int sp0 = 0; sp0 < splits; sp0 += 4) {
            f32x4_t t[4][RT];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int i = 0; i < RT; ++i)
                t[u][i] = load_agent_x4(
                    a.part, (int)((base + (int64_t)min(sp0 + u, splits - 1) * TILE_F + ((c * RT + i) * 32 + l32) * 4) * 4));
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (sp0 + u < splits)
#pragma unroll
                for (int i = 0; i < RT; ++i) acc[i][c] += t[u][i];
          }
      }
    if (tid == 0) __hip_atomic_store(a.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    prefetch_h();
  }

  // 1/rms of the rows (the same fixed order as the other kernels: per group of 16 partials in order,
  // then the 16 groups in order), by the workgroups that run the epilogue only
  if (a.ss) {
    const int per = a.ss_tiles / 16;
    for (int it = tid; it < 16 * ROWS; it += NTH) {
      const int r = it % ROWS, grp = it / ROWS;
      const float* q = a.ss + (int64_t)grp * per * a.ss_ld + min(r, a.rows - 1);  // rows past the last: unused
      float sum = 0.f;
      for (int t = 0; t < per; ++t) sum += q[(int64_t)t * a.ss_ld];
      npart[grp * ROWS + r] = sum;
    }
    __syncthreads();
    if (tid < ROWS) {
      float s2 = 0.f;
      for (int grp = 0; grp < 16; ++grp) s2 += npart[grp * ROWS + tid];
      inv_s[tid] = 1.0f / sqrtf(s2 / a.norm_dim + a.eps);
    }
    __syncthreads();
  }

#pragma unroll
  for (int c = 0; c < NB; ++c)
    if (c % NW == wave && 8 * c < a.rows) {
      f32x4_t one[RT][1];
#pragma unroll
      for (int i = 0; i < RT; ++i) one[i][0] = acc[i][c];
      const float inv[1] = {a.ss ? inv_s[8 * c + (lane & 7)] : 1.f};
      epilogue<RT, 1, EPI>(a, one, sub_row, 8 * c, a.rows - 8 * c, inv, lane,
                           EPI == EPI_RESIDUAL ? &hpre[c / NW] : nullptr);
    }
}

// ============================================================================ weight packing

// row-major bf16 [N, K] -> streaming layout (N % 16 == 0, K % 32 == 0)
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
  launch_kernel(pack_bf16_kernel, dim3(blocks), dim3(256), 0, st, src, N, K, dst);
  return hipGetLastError();
}

// ============================================================================ planning and launch

bool skinny_shape_ok(int fmt, int K) { return fmt == FMT_INT4 ? K % 512 == 0 : K % 256 == 0; }

static size_t rowsplit_lds(int nb, int kc) { return (size_t)nb * kc * 32 + (size_t)16 * 8 * nb * 4; }
static size_t ksplit_lds(int nw, int rt, int nb) {
  // reduction slots, then up to max(threads, 16 * rows) norm partials
  return (size_t)(nw - 1) * rt * nb * 4 * 64 * 4 + (size_t)std::max(64 * nw, 16 * 8 * nb) * 4;
}

#ifndef CBD_KS_MAX_UC
#define CBD_KS_MAX_UC 4
#endif
#ifndef CBD_KS_WAVE_TARGET
#define CBD_KS_WAVE_TARGET 1024
#endif
#ifndef CBD_RS_MIN_BLOCKS
#define CBD_RS_MIN_BLOCKS 600
#endif
#ifndef CBD_KS_INT4_MAX_NB
#define CBD_KS_INT4_MAX_NB 2
#endif
#ifndef CBD_KS_MAX_NB
#define CBD_KS_MAX_NB 8
#endif
#ifndef CBD_DENSE_MIN_ROWS
#define CBD_DENSE_MIN_ROWS 32
#endif
#ifndef CBD_DENSE_WG_TARGET
#define CBD_DENSE_WG_TARGET 768
#endif
#ifndef CBD_DENSE_MAX_SPLITS
#define CBD_DENSE_MAX_SPLITS 8
#endif
#ifndef CBD_DENSE_MIN_SPLIT_K
#define CBD_DENSE_MIN_SPLIT_K 1024
#endif
#ifndef CBD_DENSE1_MIN_ROWS
#define CBD_DENSE1_MIN_ROWS 16
#endif
#ifndef CBD_DENSE1_WG_TARGET
#define CBD_DENSE1_WG_TARGET 768
#endif
#ifndef CBD_DENSE_WIDE_DECODE
#define CBD_DENSE_WIDE_DECODE 1
#endif
#ifndef CBD_DENSE_WIDE_PREFILL
#define CBD_DENSE_WIDE_PREFILL 1
#endif
#ifndef CBD_DENSE_MIN_TILES
#define CBD_DENSE_MIN_TILES 40
#endif
#ifndef CBD_DENSE1_MIN_SPLIT_K
#define CBD_DENSE1_MIN_SPLIT_K 512
#endif

#ifndef CBD_WIDE_KS
#define CBD_WIDE_KS 1
#endif
#ifndef CBD_KS_MIXED_SPLIT
#define CBD_KS_MIXED_SPLIT 1
#endif
#ifndef CBD_KS_MAX_SPLITS
#define CBD_KS_MAX_SPLITS 4
#endif

namespace {
int g_plan_units = 256;  // compute units of the device the plans are for (set by the context)
}
void set_plan_compute_units(int units) {
  if (units > 0) g_plan_units = units;
}
int plan_compute_units() { return g_plan_units; }
#ifndef CBD_WIDE_MIN_ROWS
#define CBD_WIDE_MIN_ROWS 8
#endif
#ifndef CBD_WIDE_WG_TARGET
#define CBD_WIDE_WG_TARGET 256
#endif
#ifndef CBD_WIDE_MAX_SPLITS
#define CBD_WIDE_MAX_SPLITS 16
#endif
#ifndef CBD_WIDE_MIN_SPLIT_K
#define CBD_WIDE_MIN_SPLIT_K 512
#endif
#ifndef CBD_WIDE_ALL
#define CBD_WIDE_ALL 0
#endif
#ifndef CBD_WIDE_UC8
#define CBD_WIDE_UC8 1
#endif
#ifndef CBD_DENSE_WIDE_MIN_TILES
#define CBD_DENSE_WIDE_MIN_TILES 384
#endif
#ifndef CBD_WIDE_UC
#define CBD_WIDE_UC 2
#endif

SkinnyPlan plan_skinny(int epi, int fmt, int N, int K, int rows, int x_blocks, int force) {
  SkinnyPlan p{};
  // wide k split for decode steps of more than CBD_WIDE_MIN_ROWS rows (bf16 weights): 64-row tiles
  // of 4 waves, K split over workgroups up to CBD_WIDE_WG_TARGET workgroups with at least
  // CBD_WIDE_MIN_SPLIT_K inputs per split. The plan fields: rt = 4 subtiles per wave, nb = activation
  // groups (2, 4 or 8), uc = 32-input fragments per pipeline stage, waves = 4.
  const int wide_groups = (rows + 7) / 8;
  const int wide_nb = wide_groups <= 2 ? 2 : wide_groups <= 4 ? 4 : 8;
  const long n_all = epi == EPI_SWIGLU ? 2L * N : (long)N;  // weight rows
  // measured at the 8B shape: at 9..16 rows it beats the k-split kernel on long K (down), at 17..32
  // rows the k-split and dense kernels on long-K and wide products (down, gate/up, lm_head), at
  // 33..64 rows on the 4096-row products (O, down)
  const bool wide_pick = CBD_WIDE_ALL ? wide_nb >= 2
                         : wide_nb == 2 ? K >= 8192
                         : wide_nb == 4 ? (K >= 8192 || n_all >= 16384)
                                        : n_all <= 4096;
  if (force == 0 && CBD_WIDE_KS && fmt == FMT_BF16 && x_blocks == 1 && rows > CBD_WIDE_MIN_ROWS && rows <= 64 &&
      wide_pick && (epi == EPI_SWIGLU ? N % 32 == 0 : N % 64 == 0)) {  // (whole tiles at 4 subtiles, so at 2)
    p.kind = 3;
    // 33..64 rows: 2 subtiles per wave on short K (O: 22.1 -> 18.4 us per layer at B = 64; two waves
    // per SIMD instead of one), 4 on long K (down: 41.8 against 45.1 us with 2)
    p.rt = (wide_nb == 8 && K < 8192) ? 2 : 4;
    p.waves = 4;
    p.nb = wide_nb;
    p.uc = p.nb == 8 ? CBD_WIDE_UC8 : CBD_WIDE_UC;
    p.row_blocks = epi == EPI_SWIGLU ? N / (8 * p.rt) : N / (16 * p.rt);
    p.splits = 1;
    const int unit = 4 * 32 * p.uc;  // inputs of one stage of the 4 waves
    if (K % (2 * unit) == 0) {
      for (int s = 2; s <= CBD_WIDE_MAX_SPLITS; ++s)
        if (K % (s * 2 * unit) == 0 && K / s >= CBD_WIDE_MIN_SPLIT_K && (long)p.row_blocks * s <= CBD_WIDE_WG_TARGET)
          p.splits = s;
      return p;
    }
    p = SkinnyPlan{};
  }
  // dense tiles for many activation rows (bf16 weights; N in whole tiles). Prefill: 256 x 128
  // tiles of 64 x 64 waves (CBD_DENSE_WIDE_PREFILL; 128 x 128 tiles of 64 x 32 waves where N does
  // not divide). Decode steps: one activation tile of 64 rows above CBD_DENSE_MIN_ROWS rows, 32 rows
  // above CBD_DENSE1_MIN_ROWS, 128 weight rows, K split over workgroups to fill the chip; only for
  // products with enough weight tiles, or long K, to fill the chip without many splits (the others
  // measured faster on the k-split kernel). The plan fields: rt = waves along N, nb = activation
  // groups per wave, waves = all waves of the workgroup.
  auto ntiles = [&](int tn_rows) { return epi == EPI_SWIGLU ? N / (tn_rows / 2) : N / tn_rows; };
  auto divides = [&](int tn_rows) { return epi == EPI_SWIGLU ? N % (tn_rows / 2) == 0 : N % tn_rows == 0; };
  const bool dense_decode =
      rows > CBD_DENSE_MIN_ROWS ? (ntiles(128) >= CBD_DENSE_MIN_TILES || K >= 8192)
                                : (rows > CBD_DENSE1_MIN_ROWS && ntiles(128) >= CBD_DENSE_MIN_TILES && ntiles(128) <= 512);
  if (force == 0 && fmt == FMT_BF16 && K % 64 == 0 && (x_blocks > 1 || dense_decode) && divides(128)) {
    p.kind = 2;
    p.uc = 1;
    p.splits = 1;
    if (x_blocks > 1) {
      const bool wide_tile = CBD_DENSE_WIDE_PREFILL && divides(256);
      p.rt = wide_tile ? 4 : 2;
      p.nb = wide_tile ? 8 : 4;
      p.waves = 8;
      p.row_blocks = ntiles(64 * p.rt);
    } else {
      const bool wide = rows > CBD_DENSE_MIN_ROWS;
      // 256-row tiles only where they need no K split (their partial tiles are twice as large)
      const bool wide_tile = wide && CBD_DENSE_WIDE_DECODE && divides(256) && ntiles(256) >= CBD_DENSE_WIDE_MIN_TILES;
      p.rt = wide_tile ? 4 : 2;
      p.nb = wide_tile ? 8 : 4;
      p.waves = wide_tile ? 4 : wide ? 4 : 2;
      p.row_blocks = ntiles(64 * p.rt);
      const long wg_target = wide ? CBD_DENSE_WG_TARGET : CBD_DENSE1_WG_TARGET;
      const int min_k = wide ? CBD_DENSE_MIN_SPLIT_K : CBD_DENSE1_MIN_SPLIT_K;
      // most splits keeping at most wg_target workgroups and min_k inputs per split: every split
      // adds a partial tile (32 KB, or 16 KB for 32 rows) that one workgroup reads back at the end
      for (int s = 2; s <= CBD_DENSE_MAX_SPLITS; ++s)
        if (K % (64 * s) == 0 && K / s >= min_k && (long)p.row_blocks * s <= wg_target) p.splits = s;
    }
    return p;
  }
  const int per_block = x_blocks > 1 ? 64 : rows;
  const int groups = (per_block + 7) / 8;  // 8-row groups, rounded up to 1, 2, 4 or 8
  p.nb = groups <= 1 ? 1 : groups <= 2 ? 2 : groups <= 4 ? 4 : 8;
  const int step = fmt == FMT_INT4 ? 128 : 32;
  // k split: one 16*rt-row tile per workgroup, enough waves to cover the chip
  // int4 stages carry 8x more activation bytes than weight bytes per subtile: a wave takes two
  // subtiles per activation load (for SwiGLU, as for bf16: one gate, one up)
  const int ks_rt = (epi == EPI_SWIGLU || fmt == FMT_INT4) ? 2 : 1;
  const int ks_tiles = epi == EPI_SWIGLU ? N / (8 * ks_rt) : N / (16 * ks_rt);
  int ks_uc = fmt == FMT_INT4 ? 1 : (K % (4 * 128) == 0 ? 4 : (K % (4 * 64) == 0 ? 2 : 1));
  ks_uc = std::min(ks_uc, p.nb >= 8 ? 1 : p.nb >= 4 ? 2 : CBD_KS_MAX_UC);  // registers for the stages
  const int ks_unit = step * ks_uc;
  const int ks_maxw = (ks_rt == 1 && p.nb == 1) ? 16 : (fmt == FMT_INT4 && p.nb > 1) ? 4 : 8;
  const bool ks_ok = x_blocks == 1 && p.nb <= (fmt == FMT_INT4 ? CBD_KS_INT4_MAX_NB : CBD_KS_MAX_NB) &&
                     K % (4 * ks_unit) == 0 &&
                     (epi == EPI_SWIGLU ? N % (8 * ks_rt) == 0 : N % (16 * ks_rt) == 0);
  // row split: 4 waves x rt subtiles
  const int rs_rt = (epi == EPI_SWIGLU || N % 128 == 0) ? 2 : 1;
  const int rs_blocks = epi == EPI_SWIGLU ? N / 64 : N / (64 * rs_rt);
  bool use_ks = ks_ok && (long)rs_blocks < CBD_RS_MIN_BLOCKS;
  if (force < 0) use_ks = ks_ok;
  if (force > 0) use_ks = false;
  if (use_ks) {
    p.kind = 1;
    p.rt = ks_rt;
    p.uc = ks_uc;
    p.row_blocks = ks_tiles;
    p.splits = 1;
    p.kc = 0;
    // each wave needs >= 2 stages of its K slice (the loop keeps two in flight)
    // (int4 at one row group: two waves per tile to start with, so wide products stay within one
    // round of resident waves; their stages carry the dequantization and are fewer per wave)
    int nw = (fmt == FMT_INT4 && p.nb == 1) ? 2 : 4;
    if (force < 0) {
      nw = -force;
    } else {
      while (nw > 1 && K / nw < 2 * ks_unit) nw /= 2;
      while (nw < ks_maxw && (long)ks_tiles * nw < CBD_KS_WAVE_TARGET && K % (2 * nw * ks_unit) == 0 &&
             K / (2 * nw) >= 2 * ks_unit)
        nw *= 2;
    }
    // Fewer tiles than compute units leave units idle: K is then split over s workgroups per tile
    // (the same waves each, over 1/s of K), doubling s while the workgroups still fit one per unit.
    // (Splits that only even out 1.5 or 3.5 tiles per unit measured slower: the merge costs more.)
    if (force == 0) {
      const int units = plan_compute_units();
      while ((long)ks_tiles * p.splits * 2 <= units && p.splits * 2 <= CBD_KS_MAX_SPLITS &&
             K % (p.splits * 2 * nw * ks_unit) == 0 && K / (p.splits * 2 * nw) >= 2 * ks_unit)
        p.splits *= 2;
    }
    // Tiles a whole number of units plus half a unit (QKV: 384 on 256 units, gate/up: 896) leave half
    // the units one tile more than the others: the last half-unit of tiles is split in two instead,
    // so that every unit gets the same inputs and only those tiles pay the merge (8B shape, B = 8:
    // gate/up 40.5 -> 39.5 us, QKV 13.6 -> 13.2 us; B = 16 +1.5%). Not for int4 weights, whose
    // shorter streams do not repay the merge (Mistral-7B gate/up 21.7 -> 22.5 us).
    if (force == 0 && CBD_KS_MIXED_SPLIT && fmt == FMT_BF16 && p.splits == 1) {
      const int units = plan_compute_units();
      if (ks_tiles > units && ks_tiles % units == units / 2 && K % (2 * nw * ks_unit) == 0 &&
          K / (2 * nw) >= 2 * ks_unit) {
        p.splits = 2;
        p.split_from = ks_tiles - units / 2;
      }
    }
    while (fmt == FMT_BF16 && p.uc > 1 && K / (nw * p.splits) < 2 * step * p.uc) p.uc /= 2;
    p.waves = nw;
    return p;
  }
  p.kind = 0;
  p.rt = rs_rt;
  p.row_blocks = rs_blocks;
  p.uc = fmt == FMT_INT4 ? 1 : (p.nb > 2 ? 2 : 4);
  p.waves = 4;
  const int unit = step * p.uc;
  const int kc_max = std::max(unit, (2048 / p.nb) / unit * unit);  // activation chunk: LDS <= 64 KB
  if (force > 0) {
    p.splits = force;
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

template <int RT, int EPI, int FMT, int UC>
static hipError_t launch_rs(const SkinnyArgs& a, const SkinnyPlan& p, int x_blocks, hipStream_t st) {
  const dim3 grid(p.row_blocks, p.splits, x_blocks);
  const size_t lds = rowsplit_lds(p.nb, p.kc);
  switch (p.nb) {  // 8-row groups: 1, 2, 4 or 8 (the plan rounds up)
    case 1: launch_kernel((rowsplit_gemm_kernel<RT, 1, EPI, FMT, UC>), grid, dim3(256), lds, st, a); break;
    case 2: launch_kernel((rowsplit_gemm_kernel<RT, 2, EPI, FMT, UC>), grid, dim3(256), lds, st, a); break;
    case 4:
      launch_kernel((rowsplit_gemm_kernel<RT, 4, EPI, FMT, (UC > 2 ? 2 : UC)>), grid, dim3(256), lds, st, a);
      break;
    case 8:
      launch_kernel((rowsplit_gemm_kernel<RT, 8, EPI, FMT, (UC > 2 ? 2 : UC)>), grid, dim3(256), lds, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int RT, int EPI, int FMT, int UC>
static hipError_t launch_ks(const SkinnyArgs& a, const SkinnyPlan& p, hipStream_t st) {
  if (p.split_from < 0 || p.split_from > p.row_blocks || (p.split_from > 0 && p.splits < 2)) return hipErrorInvalidValue;
  const dim3 grid(p.split_from + (p.row_blocks - p.split_from) * p.splits, 1);
  if constexpr (FMT == FMT_INT4) {  // one or two 8-row groups (the plan never asks for more)
    if (p.nb == 1)
      launch_kernel((ksplit_gemm_kernel<RT, 1, EPI, FMT, UC>), grid, dim3(64 * p.waves), ksplit_lds(p.waves, RT, 1),
                    st, a, p.splits, p.split_from);
    else if (p.nb == 2)
      launch_kernel((ksplit_gemm_kernel<RT, 2, EPI, FMT, UC>), grid, dim3(64 * p.waves), ksplit_lds(p.waves, RT, 2),
                    st, a, p.splits, p.split_from);
    else
      return hipErrorInvalidValue;
  } else if (p.nb == 1) {
    launch_kernel((ksplit_gemm_kernel<RT, 1, EPI, FMT, UC>), grid, dim3(64 * p.waves), ksplit_lds(p.waves, RT, 1),
                  st, a, p.splits, p.split_from);
  } else if (p.nb == 2) {
    launch_kernel((ksplit_gemm_kernel<RT, 2, EPI, FMT, UC>), grid, dim3(64 * p.waves), ksplit_lds(p.waves, RT, 2),
                  st, a, p.splits, p.split_from);
  } else if (p.nb == 4) {
    launch_kernel((ksplit_gemm_kernel<RT, 4, EPI, FMT, (UC > 2 ? 2 : UC)>), grid, dim3(64 * p.waves),
                  ksplit_lds(p.waves, RT, 4), st, a, p.splits, p.split_from);
  } else if (p.nb == 8) {
    launch_kernel((ksplit_gemm_kernel<RT, 8, EPI, FMT, 1>), grid, dim3(64 * p.waves), ksplit_lds(p.waves, RT, 8),
                  st, a, p.splits, p.split_from);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int EPI>
static hipError_t dispatch(const SkinnyArgs& a, int fmt, int x_blocks, const SkinnyPlan& p, hipStream_t st) {
  if (p.kind == 1) {
    constexpr int KRT = EPI == EPI_SWIGLU ? 2 : 1;
    if (fmt == FMT_INT4) return launch_ks<2, EPI, FMT_INT4, 1>(a, p, st);
    if (p.uc == 4) return launch_ks<KRT, EPI, FMT_BF16, 4>(a, p, st);
    if (p.uc == 2) return launch_ks<KRT, EPI, FMT_BF16, 2>(a, p, st);
    return launch_ks<KRT, EPI, FMT_BF16, 1>(a, p, st);
  }
  if constexpr (EPI == EPI_SWIGLU) {
    if (fmt == FMT_INT4) return launch_rs<2, EPI, FMT_INT4, 1>(a, p, x_blocks, st);
    if (p.uc == 4) return launch_rs<2, EPI, FMT_BF16, 4>(a, p, x_blocks, st);
    return launch_rs<2, EPI, FMT_BF16, 2>(a, p, x_blocks, st);
  } else {
    if (p.rt == 1) {
      if (fmt == FMT_INT4) return launch_rs<1, EPI, FMT_INT4, 1>(a, p, x_blocks, st);
      if (p.uc == 4) return launch_rs<1, EPI, FMT_BF16, 4>(a, p, x_blocks, st);
      return launch_rs<1, EPI, FMT_BF16, 2>(a, p, x_blocks, st);
    }
    if (fmt == FMT_INT4) return launch_rs<2, EPI, FMT_INT4, 1>(a, p, x_blocks, st);
    if (p.uc == 4) return launch_rs<2, EPI, FMT_BF16, 4>(a, p, x_blocks, st);
    return launch_rs<2, EPI, FMT_BF16, 2>(a, p, x_blocks, st);
  }
}

hipError_t launch_skinny_gemm(SkinnyArgs a, int epi, int fmt, int x_blocks, const SkinnyPlan& p, hipStream_t st) {
  const int step = fmt == FMT_INT4 ? 128 : 32;
  if (p.kind == 2) {
    // p.rt x (waves / p.rt) waves of 64 weight rows x 8 p.nb activation rows (see plan_skinny)
    const int wn = p.rt, wm = p.waves / std::max(1, p.rt), nbw = p.nb;
    const int tm_rows = 8 * nbw * wm;
    const bool known = (wn == 4 && wm == 2 && nbw == 8) || (wn == 4 && wm == 1 && nbw == 8) ||
                       (wn == 2 && wm == 4 && nbw == 4) ||
                       (wn == 2 && wm == 2 && nbw == 4) || (wn == 2 && wm == 1 && nbw == 4);
    if (fmt != FMT_BF16 || a.rows < 1 || p.row_blocks < 1 || !known || p.waves != wn * wm || p.splits < 1 ||
        a.K % (64 * p.splits) || (p.splits > 1 && (x_blocks > 1 || a.rows > tm_rows || !a.part || !a.counters)))
      return hipErrorInvalidValue;
    const int tiles_m = (a.rows + tm_rows - 1) / tm_rows;
    dim3 grid;
    if (p.splits > 1) {
      grid = dim3(p.row_blocks * p.splits);  // (tile, split) = (id / splits, id % splits)
    } else {
      // linear ids over 8 x 8 blocks of (N tile, M tile), a whole number of blocks per XCD
      const int supers = ((p.row_blocks + 7) / 8) * ((tiles_m + 7) / 8);
      grid = dim3(((supers + 7) / 8) * 8 * 64);
    }
    const size_t lds = dense_lds(wn, wm, nbw);
    const int tn = p.row_blocks, sp = p.splits;
    const dim3 block(64 * p.waves);
    auto go = [&](auto kernel) { launch_kernel(kernel, grid, block, lds, st, a, tn, sp); };
    if (wn == 4 && wm == 2) {
      if (epi == EPI_SWIGLU) go(dense_gemm_kernel<EPI_SWIGLU, 4, 2, 8>);
      else if (epi == EPI_RESIDUAL) go(dense_gemm_kernel<EPI_RESIDUAL, 4, 2, 8>);
      else go(dense_gemm_kernel<EPI_STORE, 4, 2, 8>);
    } else if (wn == 4) {
      if (epi == EPI_SWIGLU) go(dense_gemm_kernel<EPI_SWIGLU, 4, 1, 8>);
      else if (epi == EPI_RESIDUAL) go(dense_gemm_kernel<EPI_RESIDUAL, 4, 1, 8>);
      else go(dense_gemm_kernel<EPI_STORE, 4, 1, 8>);
    } else if (wm == 4) {
      if (epi == EPI_SWIGLU) go(dense_gemm_kernel<EPI_SWIGLU, 2, 4, 4>);
      else if (epi == EPI_RESIDUAL) go(dense_gemm_kernel<EPI_RESIDUAL, 2, 4, 4>);
      else go(dense_gemm_kernel<EPI_STORE, 2, 4, 4>);
    } else if (wm == 2) {
      if (epi == EPI_SWIGLU) go(dense_gemm_kernel<EPI_SWIGLU, 2, 2, 4>);
      else if (epi == EPI_RESIDUAL) go(dense_gemm_kernel<EPI_RESIDUAL, 2, 2, 4>);
      else go(dense_gemm_kernel<EPI_STORE, 2, 2, 4>);
    } else {
      if (epi == EPI_SWIGLU) go(dense_gemm_kernel<EPI_SWIGLU, 2, 1, 4>);
      else if (epi == EPI_RESIDUAL) go(dense_gemm_kernel<EPI_RESIDUAL, 2, 1, 4>);
      else go(dense_gemm_kernel<EPI_STORE, 2, 1, 4>);
    }
    return hipGetLastError();
  }
  if (p.kind == 3) {
    const int unit = 4 * 32 * p.uc;
    const bool known = (p.nb == 2 && p.uc == CBD_WIDE_UC && p.rt == 4) || (p.nb == 4 && p.uc == CBD_WIDE_UC && p.rt == 4) ||
                       (p.nb == 8 && p.uc == CBD_WIDE_UC8 && (p.rt == 2 || p.rt == 4));
    if (fmt != FMT_BF16 || x_blocks != 1 || !known || p.waves != 4 || a.rows < 1 || a.rows > 8 * p.nb ||
        p.splits < 1 || a.K % (p.splits * unit) || a.K / p.splits < 2 * unit || p.row_blocks < 1 ||
        p.row_blocks != (epi == EPI_SWIGLU ? a.N / (8 * p.rt) : a.N / (16 * p.rt)) || (p.splits > 1 && (!a.part || !a.counters)))
      return hipErrorInvalidValue;
    const dim3 grid(p.row_blocks * p.splits), block(64 * kWideWaves);
    const size_t lds = wide_lds(p.nb, p.rt);
    auto go = [&](auto kernel) { launch_kernel(kernel, grid, block, lds, st, a, p.splits); };
    auto by_nb = [&](auto epi_c) {
      constexpr int E = decltype(epi_c)::value;
      if (p.nb == 2) go(wide_ksplit_kernel<E, 2, CBD_WIDE_UC, 4>);
      else if (p.nb == 4) go(wide_ksplit_kernel<E, 4, CBD_WIDE_UC, 4>);
      else if (p.rt == 2) go(wide_ksplit_kernel<E, 8, CBD_WIDE_UC8, 2>);
      else go(wide_ksplit_kernel<E, 8, CBD_WIDE_UC8, 4>);
    };
    if (epi == EPI_SWIGLU) by_nb(std::integral_constant<int, EPI_SWIGLU>{});
    else if (epi == EPI_RESIDUAL) by_nb(std::integral_constant<int, EPI_RESIDUAL>{});
    else by_nb(std::integral_constant<int, EPI_STORE>{});
    return hipGetLastError();
  }
  if (p.kind == 1) {
    if (x_blocks != 1 || p.nb > 8 || p.waves < 1 || p.waves > 16 || p.splits < 1 || a.K % (p.waves * p.splits) ||
        (a.K / (p.waves * p.splits)) % (step * p.uc) || (p.waves > 8 && (p.rt != 1 || p.nb != 1)) ||
        (fmt == FMT_INT4 && p.nb > 1 && p.waves > 4) || a.K / (p.waves * p.splits) < 2 * step * p.uc ||
        (p.splits > 1 && (!a.part || !a.counters)))
      return hipErrorInvalidValue;
  } else {
    if (p.splits < 1 || a.K % p.splits || (x_blocks > 1 && p.splits > 1)) return hipErrorInvalidValue;
    const int kr = a.K / p.splits;
    if (kr % p.kc || p.kc % (step * p.uc)) return hipErrorInvalidValue;
    if (p.splits > 1 && (!a.part || !a.counters)) return hipErrorInvalidValue;
    a.kc = p.kc;
  }
  if (epi == EPI_SWIGLU) return dispatch<EPI_SWIGLU>(a, fmt, x_blocks, p, st);
  if (epi == EPI_RESIDUAL) return dispatch<EPI_RESIDUAL>(a, fmt, x_blocks, p, st);
  return dispatch<EPI_STORE>(a, fmt, x_blocks, p, st);
}

}  // namespace cbd
