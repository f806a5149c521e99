// smoe_route_topk: router logits, top-k expert IDs and softmax weights.
//
// Specter paper, Incremental Routing Pattern Analyzer paragraphs (the draft
// router's top-k IDs per token and layer) and expert-wise verification
// paragraphs (the target router's routing decisions); the router stays in
// full precision (hybrid-precision layout; design notes, "Speculative
// Inference Controller").
//
// One workgroup (16 waves) per tile of `tt` tokens. The x tile is staged in
// LDS as float32; each wave owns experts e = wave, wave+16, ... and forms
// the float32 dot product in the stated order: lane l keeps the partial sum
// of the terms h = 64c + l for c = 0, 1, ... (multiply and add rounded
// separately, contraction disabled), then the halving tree
// p[l] += p[l + off], off = 32 .. 1, is done with shuffles. One wave per
// token then takes the top-k by repeated wave-wide maxima of a 64-bit key
// (order-preserving float bits, then inverted expert ID, so ties go to the
// lower ID) and the softmax weights over all E logits.
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kMaxTT = 4;

struct RouteArgs {
  const _Float16* x;
  const float* w;
  const float* bias;
  const float* gate_w;
  int32_t* ids;
  float* wout;
  float* logits;
  float* gate;
  int T, H, E, k, flags, tt;
};

// Increasing map float -> uint32 with -0.0 and +0.0 sent to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
#pragma clang fp contract(off)
  extern __shared__ float smem[];
  const int t0 = blockIdx.x * a.tt;
  const int nt = min(a.tt, a.T - t0);
  const int H = a.H, E = a.E;
  float* xs = smem;                   // [tt][H]
  float* lg = smem + a.tt * H;        // [tt][E + 1]; column E = shared-gate dot
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;

  for (int i = threadIdx.x; i < nt * H; i += kRouteThreads)
    xs[i] = static_cast<float>(a.x[static_cast<size_t>(t0) * H + i]);
  __syncthreads();

  const bool want_gate = a.gate_w != nullptr && a.gate != nullptr;
  const int nrows = E + (want_gate ? 1 : 0);
  const int nc = H / kWave;
  for (int e = wave; e < nrows; e += kRouteWaves) {
    const float* wr = e < E ? a.w + static_cast<size_t>(e) * H : a.gate_w;
    float p[kMaxTT] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < nc; ++c) {
      const float wv = wr[c * kWave + lane];
#pragma unroll
      for (int q = 0; q < kMaxTT; ++q) {
        if (q < nt) {
          const float prod = xs[q * H + c * kWave + lane] * wv;
          p[q] = p[q] + prod;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kMaxTT; ++q) {
#pragma unroll
      for (int off = kWave / 2; off >= 1; off >>= 1) {
        const float other = __shfl_down(p[q], off, kWave);
        p[q] = p[q] + other;
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < kMaxTT; ++q) {
        if (q < nt) {
          float v = p[q];
          if (e < E && a.bias != nullptr) v = v + a.bias[e];
          lg[q * (E + 1) + e] = v;
        }
      }
    }
  }
  __syncthreads();

  if (wave >= nt) return;
  const int q = wave;
  const int t = t0 + q;
  const float* l = lg + q * (E + 1);

  uint64_t key[kMaxE / kWave];
#pragma unroll
  for (int i = 0; i < kMaxE / kWave; ++i) {
    const int e = lane + i * kWave;
    key[i] = e < E ? (static_cast<uint64_t>(order_key(l[e])) << 32) |
                         static_cast<uint32_t>(0xFFFFFFFFu - static_cast<uint32_t>(e))
                   : 0ull;
  }
  int my_sel = 0;
  int first = 0;
  for (int j = 0; j < a.k; ++j) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFull));
    if (j == 0) first = e;
    if (lane == j) my_sel = e;
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; ++i)
      if (lane + i * kWave == e) key[i] = 0ull;
  }

  // softmax over all E logits, evaluated at the selected experts
  const float mx = l[first];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxE / kWave; ++i) {
    const int e = lane + i * kWave;
    if (e < E) s += expf(l[e] - mx);
  }
  s = wave_sum_f(s);
  float wj = lane < a.k ? expf(l[my_sel] - mx) / s : 0.0f;
  if (a.flags & SMOE_ROUTE_RENORM) {
    const float tot = wave_sum_f(wj);
    wj = wj / tot;
  }
  if (lane < a.k) {
    a.ids[static_cast<size_t>(t) * a.k + lane] = my_sel;
    a.wout[static_cast<size_t>(t) * a.k + lane] = wj;
  }
  if (a.logits != nullptr) {
    for (int e = lane; e < E; e += kWave) a.logits[static_cast<size_t>(t) * E + e] = l[e];
  }
  if (want_gate && lane == 0) a.gate[t] = 1.0f / (1.0f + expf(-l[E]));
}

}  // namespace
}  // namespace smoe

using namespace smoe;

extern "C" smoe_status smoe_route_topk(const void* x, const float* w_router,
                                       const float* logit_bias, int T, int H, int E, int k,
                                       int flags, int32_t* topk_ids, float* topk_w,
                                       float* logits, const float* shared_gate_w,
                                       float* shared_gate, void* stream) {
  clear_error();
  SMOE_REQUIRE(T >= 0 && H > 0 && E > 0 && k > 0, SMOE_EINVAL,
               "route_topk: need T >= 0, H > 0, E > 0, k > 0 (T=%d H=%d E=%d k=%d)", T, H, E, k);
  SMOE_REQUIRE(E <= kMaxE && k <= kMaxK && k <= E, SMOE_EUNSUPPORTED,
               "route_topk: need E <= 256 and k <= min(8, E) (E=%d k=%d)", E, k);
  SMOE_REQUIRE(H % 128 == 0 && H <= 8192, SMOE_EUNSUPPORTED,
               "route_topk: H must be a multiple of 128 and at most 8192 (H=%d)", H);
  SMOE_REQUIRE((flags & ~SMOE_ROUTE_RENORM) == 0, SMOE_EINVAL, "route_topk: unknown flags %d", flags);
  SMOE_REQUIRE((shared_gate_w == nullptr) == (shared_gate == nullptr), SMOE_EINVAL,
               "route_topk: shared_gate_w and shared_gate must both be set or both NULL");
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(x && w_router && topk_ids && topk_w, SMOE_EINVAL, "route_topk: null pointer");
  SMOE_REQUIRE(static_cast<long long>(T) * k < (1ll << 24), SMOE_EUNSUPPORTED,
               "route_topk: T*k must be below 2^24");

  // Token tile: several tokens per workgroup only for long windows, so short
  // windows spread over more compute units; LDS holds tt*H + tt*(E+1) floats.
  int tt = T >= 256 ? kMaxTT : 1;
  while (tt > 1 && (tt * H + tt * (E + 1)) * 4 > 64 * 1024) --tt;
  const size_t lds = static_cast<size_t>(tt) * (H + E + 1) * sizeof(float);
  SMOE_REQUIRE(lds <= 64 * 1024, SMOE_EUNSUPPORTED, "route_topk: H too large for one token tile");

  RouteArgs a;
  a.x = static_cast<const _Float16*>(x);
  a.w = w_router;
  a.bias = logit_bias;
  a.gate_w = shared_gate_w;
  a.ids = topk_ids;
  a.wout = topk_w;
  a.logits = logits;
  a.gate = shared_gate;
  a.T = T;
  a.H = H;
  a.E = E;
  a.k = k;
  a.flags = flags;
  a.tt = tt;
  const int grid = (T + tt - 1) / tt;
  hipLaunchKernelGGL(route_kernel, dim3(grid), dim3(kRouteThreads), lds, as_stream(stream), a);
  return check_launch("route_topk");
}
