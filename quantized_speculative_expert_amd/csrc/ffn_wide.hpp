// Interface between the expert FFN entry points (ffn.hip) and the
// long-window FFN over tiled weights (ffn_wide.hip).
#pragma once

#include <stddef.h>

#include "smoe_internal.hpp"

namespace smoe {

constexpr int kWideMinSlots = 1024;  // windows of at least this many slots (T*k)
constexpr int kWideMaxSlots = 4096;  // sorted slots kept in LDS

struct WideCall {
  int fmt;                      // routed weights: 0 = INT4 (codes + scales), 1 = FP16
  int G;                        // INT4 group size
  const void* x;                // fp16 [T][H]
  int T, k, E, H, I;
  const void *wg, *wu, *wd;     // routed weights, tiled layout
  const void *sg, *su, *sd;     // their INT4 scales (tiled), or null for FP16
  int Is;                       // shared intermediate size (0 = none)
  const void *swg, *swu, *swd;  // shared FP16 weights, tiled layout
  const int32_t* sorted_slots;  // [T*k]
  const int32_t* offsets;       // [E+1]
  void* h;                      // fp16 h of the routed positions [T*k][I], then shared [T][Is]
  float* slot_out;              // [T*k][H]
  float* shared_out;            // [T][H] or null
};

// Bytes of the h region (256-byte multiple).
size_t wide_h_bytes(long long T, long long k, long long I, long long Is);

// Whether the long-window FFN takes a call of these shapes (tiled weights
// are the caller's check).
bool wide_applicable(const WideCall& c);

// Enqueue its two launches on `st` (arguments already checked).
smoe_status wide_ffn(const WideCall& c, hipStream_t st, const char* who);

}  // namespace smoe
