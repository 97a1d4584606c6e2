// Internal launch interface between the host runtime and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace cbd {

enum { EPI_STORE = 0, EPI_RESIDUAL = 1, EPI_SWIGLU = 2 };
enum { FMT_BF16 = 0, FMT_INT4 = 1 };

// y = W x over up to three weight matrices stacked along the output dim.
struct SkinnyArgs {
  const uint16_t* x;   // bf16 activations, row stride ldx; rows padded to the column block
  int32_t ldx;
  int32_t K;
  int32_t rows;        // valid activation rows (all column blocks together)
  int32_t N;           // output features (SWIGLU: ffn width; gate = segment 0, up = segment 1)
  const void* w[3];    // per segment: bf16 [n_s, K] or int4 packed words
  const void* aux[3];  // int4: (scale, bias) pairs [K/64, n_s, 2]
  int32_t seg_end[3];  // cumulative row ends of the segments
  float* out;          // STORE / RESIDUAL: fp32 [rows, ldo] (RESIDUAL adds into it)
  uint16_t* out_bf16;  // SWIGLU: bf16 [rows, ldo]
  int32_t ldo;
};

bool skinny_shape_ok(int fmt, int K);
// x_blocks > 1: activations come in blocks of 64 rows (prefill); else one block of `rows`.
hipError_t launch_skinny_gemm(const SkinnyArgs& a, int epi, int fmt, int x_blocks, hipStream_t st);

// embed + RMSNorm: h[r] = E[tok[r]] (fp32), xn[r] = bf16(rmsnorm(h[r]) * g)
hipError_t launch_embed_norm(const int32_t* tokens, int rows, const uint16_t* embed, int vocab, int d,
                             const uint16_t* gain, float eps, float* h, uint16_t* xn, hipStream_t st);
// xn[r] = bf16(rmsnorm(h[src(r)]) * g); src = row_idx[r] if row_idx else r
hipError_t launch_rmsnorm(const float* h, const int32_t* row_idx, int rows, int d, const uint16_t* gain, float eps,
                          uint16_t* xn, hipStream_t st);
// RoPE q in place (fp32) and write rotated k, v (bf16) to each row's slab at its position
hipError_t launch_rope_append(float* qkv, int ld_qkv, const RowMeta* meta, int rows, int n_heads, int n_kv_heads,
                              int head_dim, int layer, uint8_t* arena, const float* rope_cs, hipStream_t st);
// attention of each item's query row over its key range; direct bf16 output or partials
hipError_t launch_attention(const float* qkv, int ld_qkv, const RowMeta* meta, const AttnItem* items, int n_items,
                            int n_heads, int n_kv_heads, int head_dim, int layer, const uint8_t* arena,
                            uint16_t* out, int ld_out, float* part_o, float* part_ml, int max_parts,
                            hipStream_t st);
// merge split partials of each (row, head) -> bf16 out
hipError_t launch_attn_combine(const float* part_o, const float* part_ml, const int32_t* row_parts, int rows,
                               int n_heads, int head_dim, int max_parts, uint16_t* out, int ld_out, hipStream_t st);
// greedy argmax per row, lowest id on ties
hipError_t launch_argmax(const float* logits, int rows, int vocab, int32_t* out, hipStream_t st);
// scatter canonical K/V [L, n, Hkv, Dh] into a slab at [pos, pos+n), or gather back
hipError_t launch_slab_copy(uint8_t* arena, int64_t slab_off, int cap, int pos, int n, int n_layers, int n_kv_heads,
                            int head_dim, const uint16_t* k_in, const uint16_t* v_in, uint16_t* k_out,
                            uint16_t* v_out, hipStream_t st);

}  // namespace cbd
