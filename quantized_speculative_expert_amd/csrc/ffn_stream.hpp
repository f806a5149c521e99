// Interface between the expert FFN entry points (ffn.hip) and the
// short-window streaming FFN over tiled weights (ffn_stream.hip).
#pragma once

#include <stddef.h>

#include "smoe_internal.hpp"

namespace smoe {

// stream_ffn's answer for a call outside its limits (the caller then runs
// the general kernel); not a status any entry point returns.
constexpr smoe_status kStreamNotApplicable = 1;

struct StreamCall {
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

// Bytes of the h region for a window (256-byte multiple).
size_t stream_h_bytes(long long T, long long k, long long I, long long Is);

// Enqueue the two launches of the streaming FFN on `st`, or return
// kStreamNotApplicable (nothing enqueued) when the window is outside its
// limits. Arguments are already checked by the caller.
smoe_status stream_ffn(const StreamCall& c, hipStream_t st, const char* who);

}  // namespace smoe
