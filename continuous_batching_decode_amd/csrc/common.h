// Shared device helpers for the gfx950 kernels of libcbd.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define CBD_DEVICE __device__ __forceinline__

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// bf16 <-> fp32 on raw bit patterns. fp32 -> bf16 rounds to nearest even.
CBD_DEVICE float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

CBD_DEVICE uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

CBD_DEVICE uint32_t pack_bf16x2(float lo, float hi) { return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16); }

CBD_DEVICE float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

CBD_DEVICE float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Activations fed to the weight-streaming products are stored fragment-major:
// fragments of 16 rows x 32 inputs (1 KB of bf16), fragment (row/16, k/32)
// at index (row/16) * (K/32) + k/32, and inside it lane l = 16*((k%32)/8) +
// row%16 holds 8 consecutive inputs. A wave then loads an MFMA operand of 16
// rows x 32 inputs as 1 KB of consecutive memory.
CBD_DEVICE int64_t xfrag_off(int row, int k, int K) {
  return ((int64_t)(row >> 4) * (K >> 5) + (k >> 5)) * 512 + ((((k & 31) >> 3) << 4) + (row & 15)) * 8 + (k & 7);
}

// Per-query-row metadata shared by the RoPE/append and attention kernels.
struct RowMeta {
  int64_t slab_off;  // byte offset of the row's slab in the arena
  int32_t cap;       // slab capacity (tokens)
  int32_t pos;       // position of this query token (t_s for decode, p for prefill)
};

// One attention work item: query row `row` over keys [k_begin, k_end) of its slab.
struct AttnItem {
  int32_t row;
  int32_t k_begin;
  int32_t k_end;
  int32_t part;  // partial-result slot, or -1 when the item covers all keys [0, pos]
};
