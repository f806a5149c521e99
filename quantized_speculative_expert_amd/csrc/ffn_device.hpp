// Device helpers of the expert FFN kernel (ffn.hip): vector types, global
// loads and stores, bit casts and the table-free INT4 dequantisation.
#pragma once

#include "smoe_internal.hpp"

namespace smoe {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

enum { kInt4 = 0, kFp16 = 1 };
constexpr int kBlockBytes = 64;  // bytes of one weight row per block (128 INT4 or 32 FP16 k)

// Loads and stores through global-address-space pointers. A generic pointer
// (one that went through an integer, say) would make the compiler emit flat
// instructions, which count against the LDS counter too: every LDS wait
// would then also wait for every weight load in flight.
template <typename T>
__device__ __forceinline__ T gload(const void* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}
template <typename T>
__device__ __forceinline__ void gstore(void* p, T v) {
  *(__attribute__((address_space(1))) T*)(p) = v;
}

template <typename T, typename U>
__device__ __forceinline__ T bitcast(U u) {
  static_assert(sizeof(T) == sizeof(U), "size");
  T t;
  __builtin_memcpy(&t, &u, sizeof(T));
  return t;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Eight INT4 codes of one word -> (c - 8) as fp16, in the order of its nibble positions
// 0,4,1,5,2,6,3,7 (row-major words: k order 0,4,1,5,2,6,3,7; tiled words,
// whose nibbles smoe_tile_weights stores unzipped, even k in positions 0..3
// and odd k in 4..7: natural k order).
// lo = 0x000F000F, hi = 0x00F000F0 and magic = 0x64006400 are passed in
// registers so that each mask-and-or is a single v_and_or_b32. A code in
// bits 4..7 of a half reads as 1024 + 16 c, and (1024 + 16 c) / 16 - 72 =
// c - 8 is exact in one fp16 fma, so one shift (by 8) serves all four
// pairs.
__device__ __forceinline__ f16x8 dequant_word(uint32_t w, uint32_t lo, uint32_t hi,
                                              uint32_t magic) {
  const f16x2 bias = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
  const f16x2 sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const f16x2 bias16 = {static_cast<_Float16>(-72.0f), static_cast<_Float16>(-72.0f)};
  const uint32_t w8 = w >> 8;
  const f16x2 v0 = bitcast<f16x2>((w & lo) | magic) - bias;
  const f16x2 v1 = __builtin_elementwise_fma(bitcast<f16x2>((w & hi) | magic), sixteenth, bias16);
  const f16x2 v2 = bitcast<f16x2>((w8 & lo) | magic) - bias;
  const f16x2 v3 = __builtin_elementwise_fma(bitcast<f16x2>((w8 & hi) | magic), sixteenth, bias16);
  f16x8 r;
  r[0] = v0[0]; r[1] = v0[1]; r[2] = v1[0]; r[3] = v1[1];
  r[4] = v2[0]; r[5] = v2[1]; r[6] = v3[0]; r[7] = v3[1];
  return r;
}

// Natural k order 0..7 -> 0,4,1,5,2,6,3,7 (matches dequant_word).
__device__ __forceinline__ u32x4 permute_k8(u32x4 d) {
  u32x4 e;
  e[0] = (d[0] & 0xFFFFu) | (d[2] << 16);
  e[1] = (d[0] >> 16) | (d[2] & 0xFFFF0000u);
  e[2] = (d[1] & 0xFFFFu) | (d[3] << 16);
  e[3] = (d[1] >> 16) | (d[3] & 0xFFFF0000u);
  return e;
}

}  // namespace smoe
