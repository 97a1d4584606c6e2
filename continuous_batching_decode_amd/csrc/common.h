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

// fp32 -> bf16, round to nearest even, with gfx950's packed conversion (one instruction per pair;
// non-finite inputs stay non-finite).
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
CBD_DEVICE uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{lo, hi}, bf16x2_v));
}
CBD_DEVICE uint32_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

CBD_DEVICE bf16x8_t as_frag(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// Data read once per launch (weights, K/V histories): non-temporal loads keep it from evicting
// what is reused from the caches (activations, partial tiles).
CBD_DEVICE u32x4_t load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// D += A B on a 16 x 16 x 32 bf16 tile (fp32 accumulate). Lane l supplies A row l%16 and B column
// l%16, each at k = 8*(l/16) .. 8*(l/16)+7; it receives D rows 4*(l/16) .. +3 of column l%16.
CBD_DEVICE f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Agent-scope (device-coherent) loads of 16 or 8 bytes at base + byte_off, base uniform over the
// wave: the sc1 policy makes them miss in caches that another XCD's writes do not reach, as
// __hip_atomic_load at agent scope does for 4 bytes (one request instead of four).
CBD_DEVICE f32x4_t load_agent_x4(const float* base, int byte_off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, 0x00020000);
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16));
}
CBD_DEVICE float2 load_agent_x2(const float* base, int byte_off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, 0x00020000);
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 16));
}

// Agent-scope 16- and 8-byte stores (sc1: written through to where every XCD's agent-scope loads
// read), as __hip_atomic_store at agent scope does for 4 bytes.
CBD_DEVICE void store_agent_x4(float* base, int byte_off, f32x4_t v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, byte_off, 0, 16);
}
CBD_DEVICE void store_agent_x2(float* base, int byte_off, float2 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, 0x00020000);
  typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, byte_off, 0, 16);
}

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

// Activations fed to the products are bf16 pairs (hi, lo) stored as MFMA operand fragments of
// 8 rows x 32 inputs: fragment (row/8, k/32) at index (row/8) * (K/32) + k/32, and inside it lane
// l = 16*((k%32)/8) + 8*plane + row%8 holds 8 consecutive inputs of (row, plane). One 1 KB wave
// load is a B operand whose 16 columns are the hi and lo values of 8 rows; the lo value of an
// element sits kXLo elements after its hi value.
constexpr int kXLo = 64;
CBD_DEVICE int64_t xfrag_off(int row, int k, int K) {
  return ((int64_t)(row >> 3) * (K >> 5) + (k >> 5)) * 512 + ((((k & 31) >> 3) << 4) + (row & 7)) * 8 + (k & 7);
}

// Slab layout. A sequence's slab holds, for each layer l and KV head j, a K region and a V region
// of stride * Dh bf16 elements at ((2 l + {0: K, 1: V}) * Hkv + j) * stride * Dh, where stride is
// the slab's granule-rounded capacity (a multiple of 256 tokens). Inside a region keys come in
// blocks of 32 (32 * Dh contiguous elements), each made of 1 KB MFMA operand fragments:
//  K: fragment (key half h = (key%32)/16, dim chunk u = d/32) at index h * (Dh/32) + u; in it lane
//     16 * ((d%32)/8) + key%16 holds dims d - d%8 .. +7. A fragment is the operand of a 16 x 16 x 32
//     product with keys as its 16 rows and dims as its k.
//  V: fragment t = d/16; in it lane 16 * (kk/8) + d%16 holds 8 consecutive kk, where
//     kk = 8 * ((key%16)/4) + 4 * ((key%32)/16) + key%4 reorders the block's keys. A fragment is the
//     operand with dims as rows and keys as k; the reordering matches the rows in which the score
//     tiles of keys 0..15 and 16..31 come out of the product, so probabilities feed P.V in place.
CBD_DEVICE int64_t kslab_off(int key, int d, int dh) {
  return (int64_t)(key >> 5) * 32 * dh + ((((key >> 4) & 1) * (dh >> 5) + (d >> 5)) << 9) +
         (((((d & 31) >> 3) << 4) + (key & 15)) << 3) + (d & 7);
}
CBD_DEVICE int vslab_kk(int key) { return (((key & 15) >> 2) << 3) + (((key >> 4) & 1) << 2) + (key & 3); }
CBD_DEVICE int64_t vslab_off(int key, int d, int dh) {
  const int kk = vslab_kk(key);
  return (int64_t)(key >> 5) * 32 * dh + ((d >> 4) << 9) + ((((kk >> 3) << 4) + (d & 15)) << 3) + (kk & 7);
}

// Affine 8-bit slab layout (K/V stored as codes with a float32 (scale, bias) pair per group of 64
// dims of one head vector; value = scale * code + bias). A region holds stride tokens in blocks of
// 32 keys of q8_block_bytes(Dh) bytes: 32 * Dh codes, then 32 records of Dh/64 (scale, bias) pairs.
//  codes: the fragments of the bf16 layout above with one byte per element (K: fragment
//     h * (Dh/32) + u, V: fragment t = d/16, lanes as there); 16-byte word i of lane l sits at
//     byte 1024 i + 16 l and holds fragment 2i in bytes 0..7 and fragment 2i + 1 in bytes 8..15.
//  records: key kk of the V order (vslab_kk) at byte 32 * Dh + kk * (Dh/64) * 8, group after group.
//     Lane group g = l/16 owns keys kk = 8g .. 8g + 7: exactly the keys whose scores it holds.
//
// Affine 4-bit slabs: the same blocks with 16 * Dh code bytes, two codes per byte: a fragment's 8 codes
// are 4 bytes, element e in byte e % 4, low nibble for e < 4 and high nibble for e >= 4 (so one mask
// gives elements 0..3 and a shift and mask elements 4..7, each already one per byte); 16-byte word i
// of lane l (byte 1024 i + 16 l) holds fragments 4i .. 4i + 3, fragment f at bytes 4 (f % 4) .. +3.
constexpr int kQGroup = 64;
__host__ __device__ constexpr int q_block_bytes(int dh, int bits) { return 32 * dh * bits / 8 + 32 * (dh / kQGroup) * 8; }
__host__ __device__ constexpr int q8_block_bytes(int dh) { return q_block_bytes(dh, 8); }
CBD_DEVICE int64_t kq_off(int key, int d, int dh) {
  const int f = ((key >> 4) & 1) * (dh >> 5) + (d >> 5);
  const int lane = (((d & 31) >> 3) << 4) + (key & 15);
  return (int64_t)(key >> 5) * q8_block_bytes(dh) + ((f >> 1) << 10) + (lane << 4) + ((f & 1) << 3) + (d & 7);
}
CBD_DEVICE int64_t vq_off(int key, int d, int dh) {
  const int kk = vslab_kk(key), t = d >> 4;
  const int lane = ((kk >> 3) << 4) + (d & 15);
  return (int64_t)(key >> 5) * q8_block_bytes(dh) + ((t >> 1) << 10) + (lane << 4) + ((t & 1) << 3) + (kk & 7);
}
CBD_DEVICE int64_t sbq_off(int key, int gi, int dh, int bits = 8) {
  return (int64_t)(key >> 5) * q_block_bytes(dh, bits) + 32 * dh * bits / 8 +
         ((int64_t)vslab_kk(key) * (dh / kQGroup) + gi) * 8;
}
// 4-bit codes: byte offset of (key, d); the code is in its high nibble when bit 2 of (K: d, V: kk) is set
CBD_DEVICE int64_t kq4_off(int key, int d, int dh) {
  const int f = ((key >> 4) & 1) * (dh >> 5) + (d >> 5);
  const int lane = (((d & 31) >> 3) << 4) + (key & 15);
  return (int64_t)(key >> 5) * q_block_bytes(dh, 4) + ((f >> 2) << 10) + (lane << 4) + ((f & 3) << 2) + (d & 3);
}
CBD_DEVICE int64_t vq4_off(int key, int d, int dh) {
  const int kk = vslab_kk(key), t = d >> 4;
  const int lane = ((kk >> 3) << 4) + (d & 15);
  return (int64_t)(key >> 5) * q_block_bytes(dh, 4) + ((t >> 2) << 10) + (lane << 4) + ((t & 3) << 2) + (kk & 3);
}
// Write a 4-bit code into its nibble of a byte whose other nibble another thread may be writing
// (V: keys kk and kk ^ 4 share a byte): clear and set the nibble's bits with word atomics.
CBD_DEVICE void store_nibble(uint8_t* byte_addr, int high, uint32_t code) {
  uint32_t* w = reinterpret_cast<uint32_t*>(reinterpret_cast<uintptr_t>(byte_addr) & ~uintptr_t(3));
  const int sh = 8 * (int)(reinterpret_cast<uintptr_t>(byte_addr) & 3) + 4 * high;
  atomicAnd(w, ~(15u << sh));
  atomicOr(w, (code & 15u) << sh);
}

// Affine code of x in a group with minimum lo and scale s = (max - lo) / L (q8_scale; L = 255 for 8-bit,
// 15 for 4-bit codes): the nearest grid point, decided in float32 ((x - lo) / s rounded half to even,
// clamped to 0..L); a constant group (s = 0) takes code 0.
template <int BITS = 8>
CBD_DEVICE float q8_scale(float lo, float hi) { return (hi - lo) / (float)((1 << BITS) - 1); }
template <int BITS = 8>
CBD_DEVICE uint32_t q8_code(float x, float lo, float s) {
  if (!(s > 0.f)) return 0u;
  return (uint32_t)fminf(fmaxf(rintf((x - lo) / s), 0.f), (float)((1 << BITS) - 1));
}

// Per-query-row metadata shared by the RoPE/append and attention kernels.
// A sequence forked from another one's first positions reads keys [0, pre_end) (whole blocks of 32)
// from the parent's slab (pre_off, pre_stride) and keeps the rest in its own: its slab_off is then
// shifted back by pre_end / 32 blocks, so that key k of its own part sits where the layout functions
// put key k (k >= pre_end only).
struct RowMeta {
  int64_t slab_off;  // byte offset of the row's slab in the arena (shifted as above for a fork)
  int32_t stride;    // tokens per K or V region of the slab (granule-rounded capacity)
  int32_t pos;       // position of this query token (t_s for decode, p for prefill)
  int64_t pre_off;   // the parent's slab (pre_end > 0 only)
  int32_t pre_stride;
  int32_t pre_end;   // keys below it live in the parent's slab (a multiple of 32; 0 = none)
};

// One attention work item: query row `row` (at position pos of the slab at slab_off) over keys
// [k_begin, k_end) of that slab. The slab fields repeat the row's metadata so a kernel needs one
// load to start.
struct AttnItem {
  int64_t slab_off;
  int32_t stride;
  int32_t pos;
  int32_t row;
  int32_t k_begin;
  int32_t k_end;
  int32_t part;  // partial-result slot, or -1 when the item covers all keys [0, pos]
  // prefill only: keys [0, pre_end) come from the parent's slab (decode items never straddle pre_end:
  // their slab fields already name the slab that holds their range)
  int64_t pre_off;
  int32_t pre_stride;
  int32_t pre_end;
};
