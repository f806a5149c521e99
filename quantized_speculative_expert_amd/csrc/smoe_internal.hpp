// Internal helpers shared by the libsmoe HIP sources (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smoe.h"

namespace smoe {

constexpr int kWave = 64;
constexpr int kMaxE = 256;
constexpr int kMaxK = 8;

// Thread-local text of the last failure (smoe_last_error()).
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Check the launch that was just enqueued.
smoe_status check_launch(const char* what);

// Argument checks of smoe_align_by_expert and smoe_elb_accumulate_topm
// (SMOE_OK, or the status those calls return, with the error text set).
smoe_status align_check(const int32_t* topk_ids, int T, int k, int E, const int32_t* expert_counts,
                        const int32_t* expert_offsets, const int32_t* sorted_slots,
                        const int32_t* active_experts, const int32_t* n_active);
smoe_status combine_check(const float* slot_out, const float* topk_w, int T, int k, int H,
                          const float* shared_out, const float* shared_gate, const void* y);
smoe_status elb_check(const int32_t* elb_counts, int L, int E, const int32_t* topk_ids,
                      int layer_begin, int n_layers, int T, int k, int M, const int32_t* plan_ids,
                      int flags);

#define SMOE_REQUIRE(cond, code, ...)      \
  do {                                     \
    if (!(cond)) {                         \
      ::smoe::set_error(__VA_ARGS__);      \
      return (code);                       \
    }                                      \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------------ device

// Word (of the 16 in a 64-byte INT4 block of one weight row) that the
// expert FFN's MFMA step q (0..3) of lane group g (0..3) takes, for
// quantisation groups of G = 32, 64 or 128 codes: each step's 32 codes then
// lie in one group.
__host__ __device__ constexpr int int4_word(int G, int g, int q) {
  return (q / (G / 32)) * (G / 8) + g * (G / 32) + (q % (G / 32));
}

// Lane index within the wave.
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// 64-bit mask of the lanes below the calling lane.
__device__ __forceinline__ uint64_t lanes_below_mask() {
  const int lane = lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Mask of the active lanes whose `key` (0 <= key < 256) equals ours, built
// from one ballot per key bit.
__device__ __forceinline__ uint64_t match_key8(int key, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    m &= bit ? ones : ~ones;
  }
  return valid ? m : 0ull;
}

}  // namespace smoe
