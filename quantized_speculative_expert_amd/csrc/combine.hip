// smoe_combine: routing-weighted sum of the per-slot expert outputs back in
// token order, plus the (optionally gated) shared-expert output.
//
// Specter paper, expert-wise verification paragraph: once every expert's
// sub-batch is done, each slot's output goes back to its own token, scaled
// by the router weight, and the slots of a token add up. Design notes,
// "Streamlined Execution Engine" (kernels reduce expert outputs).
//
// Streaming kernel: each thread owns 8 consecutive hidden units of one
// token (two 16-byte loads per slot, one 16-byte fp16 store).
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ slot_out, const float* __restrict__ w, int T, int k, int H,
    const float* __restrict__ shared_out, const float* __restrict__ gate,
    _Float16* __restrict__ y) {
  const int per_tok = H / 8;
  const long long idx = static_cast<long long>(blockIdx.x) * kCombineThreads + threadIdx.x;
  if (idx >= static_cast<long long>(T) * per_tok) return;
  const int t = static_cast<int>(idx / per_tok);
  const int h0 = static_cast<int>(idx % per_tok) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  // every slot's loads (and the shared row's) go out before the first is
  // used (k <= kMaxK)
  float4 sa = {0.0f, 0.0f, 0.0f, 0.0f}, sb = sa;
  float sg = 1.0f;
  if (shared_out != nullptr) {
    const float4* src = reinterpret_cast<const float4*>(shared_out + static_cast<size_t>(t) * H + h0);
    sa = src[0];
    sb = src[1];
    if (gate != nullptr) sg = gate[t];
  }
  float4 va[kMaxK], vb[kMaxK];
  float wv[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      wv[j] = w[static_cast<size_t>(t) * k + j];
      const float4* src =
          reinterpret_cast<const float4*>(slot_out + (static_cast<size_t>(t) * k + j) * H + h0);
      va[j] = src[0];
      vb[j] = src[1];
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      const float wj = wv[j];
      const float4 a = va[j], b = vb[j];
      acc[0] += wj * a.x; acc[1] += wj * a.y; acc[2] += wj * a.z; acc[3] += wj * a.w;
      acc[4] += wj * b.x; acc[5] += wj * b.y; acc[6] += wj * b.z; acc[7] += wj * b.w;
    }
  }
  if (shared_out != nullptr) {
    const float g = sg;
    const float4 a = sa, b = sb;
    acc[0] += g * a.x; acc[1] += g * a.y; acc[2] += g * a.z; acc[3] += g * a.w;
    acc[4] += g * b.x; acc[5] += g * b.y; acc[6] += g * b.z; acc[7] += g * b.w;
  }
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  h8 out;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = static_cast<_Float16>(acc[i]);
  *reinterpret_cast<h8*>(y + static_cast<size_t>(t) * H + h0) = out;
}

}  // namespace
}  // namespace smoe

using namespace smoe;

namespace smoe {
smoe_status combine_check(const float* slot_out, const float* topk_w, int T, int k, int H,
                          const float* shared_out, const float* shared_gate, const void* y) {
  SMOE_REQUIRE(T >= 0 && k > 0 && H > 0, SMOE_EINVAL,
               "combine: need T >= 0, k > 0, H > 0 (T=%d k=%d H=%d)", T, k, H);
  SMOE_REQUIRE(k <= kMaxK && H % 128 == 0, SMOE_EUNSUPPORTED,
               "combine: need k <= 8 and H a multiple of 128 (k=%d H=%d)", k, H);
  SMOE_REQUIRE(shared_gate == nullptr || shared_out != nullptr, SMOE_EINVAL,
               "combine: shared_gate given without shared_out");
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(slot_out && topk_w && y, SMOE_EINVAL, "combine: null pointer");
  SMOE_REQUIRE(aligned16(slot_out) && aligned16(y) && (!shared_out || aligned16(shared_out)),
               SMOE_EINVAL, "combine: slot_out, shared_out and y must be 16-byte aligned");
  return SMOE_OK;
}
}  // namespace smoe

extern "C" smoe_status smoe_combine(const float* slot_out, const float* topk_w, int T, int k,
                                    int H, const float* shared_out, const float* shared_gate,
                                    void* y, void* stream) {
  clear_error();
  const smoe_status st = combine_check(slot_out, topk_w, T, k, H, shared_out, shared_gate, y);
  if (st != SMOE_OK || T == 0) return st;
  const long long threads = static_cast<long long>(T) * (H / 8);
  const int grid = static_cast<int>((threads + kCombineThreads - 1) / kCombineThreads);
  hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(kCombineThreads), 0, as_stream(stream),
                     slot_out, topk_w, T, k, H, shared_out, shared_gate,
                     static_cast<_Float16*>(y));
  return check_launch("combine");
}
