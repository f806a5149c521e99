// smoe_route_topk: router logits, top-k expert IDs and softmax weights.
//
// Specter paper, Incremental Routing Pattern Analyzer paragraphs (the draft
// router's top-k IDs per token and layer) and expert-wise verification
// paragraphs (the target router's routing decisions); the router stays in
// full precision (hybrid-precision layout; design notes, "Speculative
// Inference Controller").
//
// One workgroup of 8 waves per token. The token's x row is staged in LDS as
// float32; wave w owns experts e = w, w + 8, ... and forms the float32 dot
// product in the stated order: lane l keeps the partial sum of the terms
// h = 64c + l for c = 0, 1, ... (multiply and add rounded separately,
// contraction disabled), then the halving tree p[l] += p[l + off],
// off = 32 .. 1, is done with shuffles. A wave issues the router-row loads
// of four experts (up to 32 chunks each) before using any of them, so the
// row reads overlap instead of waiting one latency per chunk. One wave then
// takes the top-k by repeated wave-wide maxima of a 64-bit key
// (order-preserving float bits, then inverted expert ID, so ties go to the
// lower ID) and the softmax weights over all E logits.
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kSlice = 32;  // chunks of 64 per load batch (2048 h)

struct RouteArgs {
  const _Float16* x;
  const float* w;
  const float* bias;
  const float* gate_w;
  int32_t* ids;
  float* wout;
  float* logits;
  float* gate;
  int T, H, E, k, flags;
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
  const int t = blockIdx.x;
  const int H = a.H, E = a.E;
  float* xs = smem;        // [H]
  float* lg = smem + H;    // [E + 1]; entry E = shared-gate dot
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;

  for (int i = threadIdx.x; i < H; i += kRouteThreads)
    xs[i] = static_cast<float>(a.x[static_cast<size_t>(t) * H + i]);
  __syncthreads();

  const bool want_gate = a.gate_w != nullptr && a.gate != nullptr;
  const int nrows = E + (want_gate ? 1 : 0);
  const int nc = H / kWave;
  auto row_ptr = [&](int e) { return e < E ? a.w + static_cast<size_t>(e) * H : a.gate_w; };
  // experts e = wave + kRouteWaves * (kPerRound * j + i), kPerRound at a time:
  // all their row loads of a slice go out before any is used
  constexpr int kPerRound = 4;
  for (int e0 = wave; e0 < nrows; e0 += kPerRound * kRouteWaves) {
    const float* wr[kPerRound];
    bool has[kPerRound];
#pragma unroll
    for (int i = 0; i < kPerRound; ++i) {
      const int e = e0 + i * kRouteWaves;
      has[i] = e < nrows;
      wr[i] = row_ptr(has[i] ? e : e0);
    }
    float p[kPerRound];
#pragma unroll
    for (int i = 0; i < kPerRound; ++i) p[i] = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += kSlice) {
      float v[kPerRound][kSlice];
#pragma unroll
      for (int j = 0; j < kSlice; ++j) {
        const int c = min(c0 + j, nc - 1);
#pragma unroll
        for (int i = 0; i < kPerRound; ++i) v[i][j] = wr[i][c * kWave + lane];
      }
#pragma unroll
      for (int j = 0; j < kSlice; ++j) {
        if (c0 + j < nc) {
          const float xv = xs[(c0 + j) * kWave + lane];
#pragma unroll
          for (int i = 0; i < kPerRound; ++i) {
            const float prod = xv * v[i][j];
            p[i] = p[i] + prod;
          }
        }
      }
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
#pragma unroll
      for (int i = 0; i < kPerRound; ++i) {
        const float o = __shfl_down(p[i], off, kWave);
        p[i] = p[i] + o;
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < kPerRound; ++i) {
        const int e = e0 + i * kRouteWaves;
        if (has[i]) {
          float v = p[i];
          if (e < E && a.bias != nullptr) v = v + a.bias[e];
          lg[e] = v;
        }
      }
    }
  }
  __syncthreads();

  if (wave != 0) return;
  const float* l = lg;

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

  const size_t lds = static_cast<size_t>(H + E + 1) * sizeof(float);

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
  hipLaunchKernelGGL(route_kernel, dim3(T), dim3(kRouteThreads), lds, as_stream(stream), a);
  return check_launch("route_topk");
}
