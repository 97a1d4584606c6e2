// Batched weight-streaming product for the decode step and its prefill.
//
// y[b, n] = sum_k W[n, k] x[b, k] for up to 64 rows b per launch column-block.
// The page "Continuous Decode Batching - the transformer capture" (section
// "The throughput law") is the reason for the shape of this kernel: the
// weight read w is paid once per launch whatever the number of rows, so the
// kernel is organised around streaming W from HBM exactly once with wide,
// coalesced loads, and every row of the batch rides on that single read.
//
// Mapping (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//  - A operand = 16 consecutive weight rows x 32 inputs (one 16-byte load
//    per lane: lane l reads row l%16, inputs 8*(l/16)..+7).
//  - B operand = 16 batch rows x the same 32 inputs of the bf16 activations.
//  - A workgroup (4 waves) owns RT row-subtiles of 16 weight rows and covers
//    the whole input dimension; each wave takes a contiguous quarter of K,
//    and the four partial sums are added in a fixed order through LDS, so the
//    result does not depend on scheduling.
//  - NB column tiles of 16 cover B <= 16*NB rows; padding rows of the
//    activation buffer only affect padding outputs (an MFMA output column
//    depends only on the same column of B), which are never stored.
// int4 weights (4-bit affine, groups of 64 inputs): codes are widened to the
// bf16 values 128+q with one and-or per pair and multiplied on the MFMA
// unit; the affine map is applied once per group and output:
//   sum_k x_k (s q_k + b) = s * sum_k x_k (128 + q_k) + (b - 128 s) * sum_k x_k,
// where sum_k x_k over the group comes from one more MFMA with an all-ones A.
#include "common.h"
#include "kernels.h"

namespace cbd {

namespace {

template <int N>
struct Frag {
  bf16x8_t v[N];
};

CBD_DEVICE bf16x8_t load_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

CBD_DEVICE bf16x8_t as_frag(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

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

// Locate the first weight row of a 16-row subtile in the concatenated segments.
CBD_DEVICE int seg_of(const SkinnyArgs& a, int grow) {
  return grow < a.seg_end[0] ? 0 : (grow < a.seg_end[1] ? 1 : 2);
}
CBD_DEVICE int seg_begin(const SkinnyArgs& a, int s) { return s == 0 ? 0 : a.seg_end[s - 1]; }

}  // namespace

template <int RT, int NB, int EPI, int FMT, int UC>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(SkinnyArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int tile = blockIdx.x;
  const int xblk = blockIdx.y;
  const int K = a.K;
  const int kw = K >> 2;  // each wave: a contiguous quarter of the inputs
  const int k0 = wave * kw;

  const uint16_t* X = a.x + (int64_t)xblk * (16 * NB) * (int64_t)a.ldx;
  const int rows_valid = min(16 * NB, a.rows - xblk * 16 * NB);

  // weight-row subtiles of this workgroup
  int sub_row[RT];   // concatenated row index of subtile i (first of 16)
  int sub_seg[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    int grow;
    if (EPI == EPI_SWIGLU) {
      // first half of the subtiles from the gate segment, second half from up
      const int half = RT / 2;
      grow = (i < half) ? tile * 16 * half + 16 * i : a.seg_end[0] + tile * 16 * half + 16 * (i - half);
    } else {
      grow = tile * 16 * RT + 16 * i;
    }
    sub_row[i] = grow;
    sub_seg[i] = seg_of(a, grow);
  }

  f32x4_t acc[RT][NB];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[i][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xr[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) xr[c] = X + (int64_t)(16 * c + r16) * a.ldx;

  if (FMT == FMT_BF16) {
    const uint16_t* wr[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int s = sub_seg[i];
      const int local = sub_row[i] - seg_begin(a, s) + r16;
      wr[i] = reinterpret_cast<const uint16_t*>(a.w[s]) + (int64_t)local * K + 8 * g;
    }
    for (int k = k0; k < k0 + kw; k += 32 * UC) {
      bf16x8_t A[UC][RT], Bv[UC][NB];
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int i = 0; i < RT; ++i) A[u][i] = load_frag(wr[i] + k + 32 * u);
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int c = 0; c < NB; ++c) Bv[u][c] = load_frag(xr[c] + k + 32 * u + 8 * g);
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int c = 0; c < NB; ++c) acc[i][c] = mfma(A[u][i], Bv[u][c], acc[i][c]);
    }
  } else {
    // int4: 128 inputs per block; lane group g reads words 4g..4g+3 of the block
    const uint32_t* wr[RT];
    const uint16_t* ar[RT];
    int seg_rows[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int s = sub_seg[i];
      const int sb = seg_begin(a, s);
      const int local = sub_row[i] - sb + r16;
      wr[i] = reinterpret_cast<const uint32_t*>(a.w[s]) + (int64_t)local * (K >> 3) + 4 * g;
      seg_rows[i] = a.seg_end[s] - sb;
      // scale/bias pairs of output rows 4*g .. 4*g+3 of the subtile
      ar[i] = reinterpret_cast<const uint16_t*>(a.aux[s]) + (int64_t)(sub_row[i] - sb + 4 * g) * 2;
    }
    const uint4 ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8_t ones = as_frag(ones_u);
    for (int k = k0; k < k0 + kw; k += 128 * UC) {
      uint4 Wq[UC][RT];
      uint4 SB[UC][RT][2];
      bf16x8_t Bv[UC][4][NB];
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int i = 0; i < RT; ++i) Wq[u][i] = *reinterpret_cast<const uint4*>(wr[i] + ((k + 128 * u) >> 3));
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int c = 0; c < NB; ++c)
            Bv[u][j][c] = load_frag(xr[c] + k + 128 * u + 64 * (j >> 1) + 16 * g + 8 * (j & 1));
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int grp = ((k + 128 * u) >> 6) + h;
            SB[u][i][h] = *reinterpret_cast<const uint4*>(ar[i] + (int64_t)grp * seg_rows[i] * 2);
          }
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4_t xs[NB];
#pragma unroll
          for (int c = 0; c < NB; ++c) {
            xs[c] = mfma(ones, Bv[u][2 * h][c], f32x4_t{0.f, 0.f, 0.f, 0.f});
            xs[c] = mfma(ones, Bv[u][2 * h + 1][c], xs[c]);
          }
#pragma unroll
          for (int i = 0; i < RT; ++i) {
            const uint32_t w0 = h ? Wq[u][i].z : Wq[u][i].x;
            const uint32_t w1 = h ? Wq[u][i].w : Wq[u][i].y;
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
              f32x4_t t = mfma(A0, Bv[u][2 * h][c], f32x4_t{0.f, 0.f, 0.f, 0.f});
              t = mfma(A1, Bv[u][2 * h + 1][c], t);
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][c][e] += sc[e] * t[e] + bc[e] * xs[c][e];
            }
          }
        }
    }
  }

  // fixed-order reduction of the four K quarters through LDS
  __shared__ float red[3][RT * NB * 4][64];
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave - 1][(i * NB + c) * 4 + e][lane] = acc[i][c][e];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][c][e] += red[w][(i * NB + c) * 4 + e][lane];

  // epilogue: lane holds y[b = 16c + l%16][n = subtile + 4*(l/16) + e]
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int b = 16 * c + r16;
    if (b >= rows_valid) continue;
    const int64_t orow = (int64_t)(xblk * 16 * NB + b) * a.ldo;
    if (EPI == EPI_SWIGLU) {
      const int half = RT / 2;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const int n = tile * 16 * half + 16 * i + 4 * g;
        const f32x4_t gt = acc[i][c], up = acc[i + half][c];
        uint2 o;
        o.x = pack_bf16x2(silu_f(gt[0]) * up[0], silu_f(gt[1]) * up[1]);
        o.y = pack_bf16x2(silu_f(gt[2]) * up[2], silu_f(gt[3]) * up[3]);
        *reinterpret_cast<uint2*>(a.out_bf16 + orow + n) = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int n = sub_row[i] + 4 * g;
        float4* p = reinterpret_cast<float4*>(a.out + orow + n);
        float4 v = make_float4(acc[i][c][0], acc[i][c][1], acc[i][c][2], acc[i][c][3]);
        if (EPI == EPI_RESIDUAL) {
          const float4 h = *p;
          v.x += h.x; v.y += h.y; v.z += h.z; v.w += h.w;
        }
        *p = v;
      }
    }
  }
}

// ----------------------------------------------------------------------------- launcher

template <int RT, int EPI, int FMT, int UC>
static hipError_t launch_nb(const SkinnyArgs& a, int nb, dim3 grid, hipStream_t st) {
  switch (nb) {
    case 1: hipLaunchKernelGGL((skinny_gemm_kernel<RT, 1, EPI, FMT, UC>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((skinny_gemm_kernel<RT, 2, EPI, FMT, UC>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((skinny_gemm_kernel<RT, 3, EPI, FMT, UC>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((skinny_gemm_kernel<RT, 4, EPI, FMT, UC>), grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

template <int RT, int EPI>
static hipError_t launch_fmt(const SkinnyArgs& a, int fmt, int nb, dim3 grid, hipStream_t st) {
  if (fmt == FMT_INT4) return launch_nb<RT, EPI, FMT_INT4, 1>(a, nb, grid, st);
  if ((a.K / 4) % 128 == 0) return launch_nb<RT, EPI, FMT_BF16, 4>(a, nb, grid, st);
  return launch_nb<RT, EPI, FMT_BF16, 2>(a, nb, grid, st);
}

bool skinny_shape_ok(int fmt, int K) { return fmt == FMT_INT4 ? K % 512 == 0 : K % 256 == 0; }

hipError_t launch_skinny_gemm(const SkinnyArgs& a, int epi, int fmt, int x_blocks, hipStream_t st) {
  // rows per column block: 16*nb with nb = ceil(min(rows, 64) / 16)
  const int per_block = x_blocks > 1 ? 64 : a.rows;
  const int nb = (per_block + 15) / 16;
  if (epi == EPI_SWIGLU) {
    dim3 grid(a.N / 16, x_blocks);
    return launch_fmt<2, EPI_SWIGLU>(a, fmt, nb, grid, st);
  }
  dim3 grid(a.N / 16, x_blocks);
  if (epi == EPI_RESIDUAL) return launch_fmt<1, EPI_RESIDUAL>(a, fmt, nb, grid, st);
  return launch_fmt<1, EPI_STORE>(a, fmt, nb, grid, st);
}

}  // namespace cbd
