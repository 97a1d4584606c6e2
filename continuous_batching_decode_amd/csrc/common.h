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
