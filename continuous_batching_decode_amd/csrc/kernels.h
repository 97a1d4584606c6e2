// Internal launch interface between the host runtime and the gfx950 kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "../../include/cbd.h"

namespace cbd {

// Record the message of a failing call (cbd_last_error) and return its status.
cbd_status record_error(cbd_status s, const char* fmt, ...);

// Profiling hook. When start is set, the next kernel launched from this thread goes through
// hipExtLaunchKernelGGL, which stamps start/stop at that kernel's own begin and end (no dispatch
// or event-packet overhead inside the interval), and the hook is cleared.
struct LaunchEvents {
  hipEvent_t start, stop;
};
LaunchEvents& launch_events();

template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st, Args... args) {
  LaunchEvents& ev = launch_events();
  if (ev.start) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev.start, ev.stop, 0, args...);
    ev = LaunchEvents{nullptr, nullptr};
  } else {
    kernel<<<grid, block, lds, st>>>(args...);
  }
}

enum { EPI_STORE = 0, EPI_RESIDUAL = 1, EPI_SWIGLU = 2 };
enum { FMT_BF16 = 0, FMT_INT4 = 1 };

// y = W x over up to three weight matrices stacked along the output dim.
// Activations come as two bf16 planes (hi, lo) in the fragment-major layout (xfrag_off).
struct SkinnyArgs {
  const uint16_t* x;       // plane 0 (hi); plane 1 (lo) at x + x_plane
  int64_t x_plane;
  int32_t K;
  int32_t rows;            // valid output rows (all column blocks together)
  int32_t N;               // output features (SWIGLU: ffn width; gate = segment 0, up = segment 1)
  const void* w[3];        // per segment: streaming-layout bf16 or int4 words
  const void* aux[3];      // int4: (scale, bias) pairs [K/64, n_s, 2]
  int32_t seg_end[3];      // cumulative row ends of the segments
  // input normalisation: accumulators *= 1/sqrt(sum_t ss[t][row] / norm_dim + eps) (ss == null: none)
  const float* ss;
  int32_t ss_tiles;        // number of 16-feature partial sums per row (a multiple of 16)
  int32_t ss_ld;
  float norm_dim;
  float eps;
  // outputs
  float* out;              // STORE: fp32 [rows, ldo]; RESIDUAL: the fp32 residual stream (in/out)
  int32_t ldo;
  uint16_t* out_x;         // SWIGLU: product planes; RESIDUAL: planes of next_gain * h (fragment-major, K = N)
  int64_t out_plane;
  const uint16_t* next_gain;  // RESIDUAL: gain of the norm that consumes h next (null: no planes)
  float* ss_out;           // RESIDUAL: partial sums of squares of h, [N/16][ss_out_ld]
  int32_t ss_out_ld;
  // split-K workspace of the row-split kernel: partial tiles and arrival counters (zero between launches)
  float* part;
  int32_t* counters;
  int32_t kc;              // activation chunk staged in LDS (set from the plan)
};

// How one launch is cut.
//  kind 0 (row split): 4 waves x rt subtiles of 16 rows per workgroup share activation
//    chunks of kc inputs staged in LDS; K split over `splits` workgroups.
//  kind 1 (k split): one tile of 16*rt rows per workgroup, its `waves` waves each stream a
//    contiguous 1/waves of K with activations read from L2; partial sums added through LDS; K split
//    over `splits` workgroups where that evens out the work per compute unit.
//  kind 2 (dense): rt x (waves / rt) waves of 64 weight rows x 8*nb activation rows per
//    workgroup, both operands staged in LDS; K split over `splits` workgroups (one activation
//    tile only).
//  kind 3 (wide k split): 4 waves x rt subtiles of 16 rows (16 rt weight rows) per workgroup, each wave
//    a quarter of the workgroup's K range with all nb activation groups (activations read from
//    L2); K split over `splits` workgroups; decode steps of 9..64 rows.
struct SkinnyPlan {
  int kind, nb, rt, uc, row_blocks, splits, kc, waves;
  int split_from;  // k split: tiles below take one workgroup (the whole K), the rest `splits` each
};

bool skinny_shape_ok(int fmt, int K);
// x_blocks > 1: activation rows come in blocks of 64 (prefill); else one block of `rows`.
// force: 0 = chosen from the shape; > 0 = row split over `force` workgroups; < 0 = k split
// over -force waves.
SkinnyPlan plan_skinny(int epi, int fmt, int N, int K, int rows, int x_blocks, int force);
// compute units the plans even the work over (the device's count; 256 until set)
void set_plan_compute_units(int units);
int plan_compute_units();
// workspace bytes a plan needs for its partial tiles
inline size_t skinny_part_bytes(const SkinnyPlan& p) {
  if (p.splits <= 1) return 0;
  if (p.kind == 2) return (size_t)p.row_blocks * p.splits * p.waves * 4 * p.nb * 32 * 4 * 4;  // hi + lo added
  if (p.kind == 3) return (size_t)p.row_blocks * p.splits * p.nb * p.rt * 32 * 4 * 4;  // hi + lo added
  if (p.kind == 1) return (size_t)p.row_blocks * p.splits * p.rt * p.nb * 4 * 64 * 4;  // raw sums
  return p.kind == 0 ? (size_t)p.row_blocks * p.splits * 4 * p.rt * p.nb * 4 * 64 * 4 : 0;
}
hipError_t launch_skinny_gemm(SkinnyArgs a, int epi, int fmt, int x_blocks, const SkinnyPlan& p, hipStream_t st);
// row-major bf16 [N, K] -> streaming layout (fragments of 16 rows x 32 inputs, lane order, along K)
hipError_t launch_pack_bf16(const uint16_t* src, int64_t N, int64_t K, uint16_t* dst, hipStream_t st);

// split fp32 rows [rows, K] into fragment-major hi/lo bf16 planes: hi = bf16(x), lo = bf16(x - hi)
hipError_t launch_split_planes(const float* x, int rows, int K, uint16_t* out, int64_t plane, hipStream_t st);
// gather activation rows (fragment-major planes, K = d) and their sums of squares into compact rows
hipError_t launch_gather_rows(const uint16_t* x, int64_t x_plane, const float* ss, int ss_ld, const int32_t* row_idx,
                              int rows, int d, uint16_t* out, int64_t out_plane, float* ss_out, int ss_out_ld,
                              hipStream_t st);

// embedding gather: h[r] = E[tok[r]] (fp32); planes of gain * h; per-16-feature sums of squares
// ss[t][r] (row stride ss_ld)
hipError_t launch_embed(const int32_t* tokens, int rows, const uint16_t* embed, int vocab, int d,
                        const uint16_t* gain, float* h, uint16_t* xplanes, int64_t plane, float* ss, int ss_ld,
                        hipStream_t st);
// RoPE q in place (fp32) and write rotated k, v (bf16) to each row's slab at its position
hipError_t launch_rope_append(float* qkv, int ld_qkv, const RowMeta* meta, int rows, int n_heads, int n_kv_heads,
                              int head_dim, int layer, uint8_t* arena, const float* rope_cs, hipStream_t st);
// the same for affine 8-bit slabs (k and v quantized per KV head and group of 64 dims)
hipError_t launch_rope_append_q8(float* qkv, int ld_qkv, const RowMeta* meta, int rows, int n_heads, int n_kv_heads,
                                 int head_dim, int layer, uint8_t* arena, const float* rope_cs, int bits,
                                 hipStream_t st);
// Attention of each item's query row over its key range of the row's slab.
struct AttnArgs {
  const float* qkv;          // projections [rows, ld_qkv]: q heads, then k heads, then v heads
  int32_t ld_qkv;
  const RowMeta* meta;
  const AttnItem* items;
  int32_t n_heads, n_kv_heads, layer;
  uint8_t* arena;
  const float2* rope_cs;     // [max_pos][head_dim/2] (cos, sin)
  uint16_t* out;             // output planes (hi; lo at out + out_plane), fragment-major with K = ld_out
  int64_t out_plane;
  int32_t ld_out;
  float* part_o;             // split partials [slot][n_heads][head_dim]
  float* part_ml;            // split (max, sum) [slot][n_heads][2]
  const int2* row_parts;     // per row: (first slot, number of splits; 0 = not split)
  int32_t* counters;         // per (row, KV head) arrival counters, zero between launches
};
// decode: q unrotated; the item ending at pos + 1 rotates the new k, appends K/V at pos and uses it;
// items cover key ranges that start at multiples of 32 (one wave per item and KV head)
hipError_t launch_decode_attention(const AttnArgs& a, int n_items, int head_dim, hipStream_t st);
// prefill: q rotated and every token's K/V appended beforehand (one workgroup per item and KV head)
hipError_t launch_prefill_attention(const AttnArgs& a, int n_items, int head_dim, hipStream_t st);
// decode over affine 8-bit slabs (same items, splits and outputs as launch_decode_attention; the
// appending item quantizes the new token's K/V into the slab)
hipError_t launch_decode_attention_q8(const AttnArgs& a, int n_items, int head_dim, int bits, hipStream_t st);
hipError_t launch_prefill_attention_q8(const AttnArgs& a, int n_items, int head_dim, int bits, hipStream_t st);

// greedy argmax per row, lowest id on ties
// part: kArgmaxSegments x 64 (max, index) pairs; counters: 64 ints, zero between launches
constexpr int kArgmaxSegments = 64;
// seeded top-p sampling: per-row parameters passed by value (rows <= 64)
struct SampleArgs {
  float temperature[64];  // 0: greedy
  float top_p[64];        // in (0, 1]
  uint64_t seed[64];      // Philox4x64-10 key word 0
  uint64_t index[64];     // counter word 0
};
// its workspace: per-row weights (bit patterns), chunk maxima and masses, byte histograms of the
// chunks for the seven levels of the two searches, tie counts, and the per-row state between launches
constexpr int kSampleChunks = 32;
struct SampleWs {
  uint32_t* bits;  // [64][vocab]
  float* pmax;     // [64][chunks]
  int32_t* pidx;   // [64][chunks]
  uint64_t* pw;    // [64][chunks]
  uint64_t* hist;  // [7][64][chunks][256]
  uint32_t* cnt;   // [2][64][chunks][256]
  uint8_t* state;  // [64] per-row records
  size_t bytes;
};
SampleWs sample_ws_layout(uint8_t* base, int vocab);  // base == nullptr: sizes only
hipError_t launch_sample_top_p(const float* logits, int rows, int vocab, const SampleArgs& p, const SampleWs& ws,
                               int32_t* out, hipStream_t st);
hipError_t launch_argmax(const float* logits, int rows, int vocab, float* part, int32_t* counters, int32_t* out,
                         hipStream_t st);
// scatter canonical K/V [L, n_all, Hkv, Dh] tokens [t_off, t_off + n) into a slab at [pos, pos+n), or
// gather them back
hipError_t launch_slab_copy(uint8_t* arena, int64_t slab_off, int stride, int pos, int n, int n_all, int t_off,
                            int n_layers, int n_kv_heads, int head_dim, const uint16_t* k_in, const uint16_t* v_in,
                            uint16_t* k_out, uint16_t* v_out, hipStream_t st);
// affine 8-bit slabs: quantize canonical bf16 K/V [L, n_all, Hkv, Dh] tokens [t_off, t_off + n) into
// [pos, pos+n) (k_in, v_in), or gather codes [L, n_all, 2, Hkv, Dh] and (scale, bias) pairs
// [L, n_all, 2, Hkv, Dh/64, 2] back (codes_out, sb_out)
hipError_t launch_slab_q8(uint8_t* arena, int64_t slab_off, int stride, int pos, int n, int n_all, int t_off,
                          int n_layers, int n_kv_heads, int head_dim, const uint16_t* k_in, const uint16_t* v_in,
                          uint8_t* codes_out, float* sb_out, int bits, hipStream_t st);

}  // namespace cbd
