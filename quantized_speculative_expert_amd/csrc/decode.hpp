// Interface between the one-call draft layer (ffn.hip) and the single-token
// draft layer over tiled weights (decode.hip).
#pragma once

#include <stddef.h>

#include "smoe_blocks.hpp"

namespace smoe {

struct DecodeCall {
  FusedArgs f;                  // routing, alignment and ELB of the one token (f.r.T == 1)
  int G, I, Is;                 // INT4 group size, routed and shared intermediate sizes
  const void *wg, *wu, *wd;     // routed INT4 codes, tiled layout
  const void *sg, *su, *sd;     // their scales, tiled
  const void *swg, *swu, *swd;  // shared FP16 weights, tiled (Is > 0)
  void* region;                 // the layer's part of the FFN workspace (256-byte aligned)
  float* slot_out;              // [k][H]
  float* shared_out;            // [H] or null (Is = 0)
  void* y;                      // fp16 [H]
};

// Bytes of the workspace region the single-token layer uses (256-byte
// multiple); the FFN workspace of a one-token window carries it after its
// own layout.
size_t decode_region_bytes(long long k, long long H, long long I, long long Is);

// Whether a layer call of these shapes takes the single-token path (tiled
// weights are the caller's check).
bool decode_applicable(int T, int k, int E, int H, int I, int Is, int G);

// Enqueue its two launches on `st` (arguments already checked).
smoe_status decode_layer(const DecodeCall& c, hipStream_t st, const char* who);

}  // namespace smoe
