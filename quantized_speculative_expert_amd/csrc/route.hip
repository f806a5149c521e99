// smoe_route_topk: router logits, top-k expert IDs and softmax weights.
//
// Specter paper, Incremental Routing Pattern Analyzer paragraphs (the draft
// router's top-k IDs per token and layer) and expert-wise verification
// paragraphs (the target router's routing decisions); the router stays in
// full precision (hybrid-precision layout; design notes, "Speculative
// Inference Controller").
//
// Two launches. The logits kernel spreads the T x E dot products over many
// workgroups: workgroup (g, j) takes router rows 8g .. 8g+7 (one per wave;
// row E is the shared-gate vector) and a tile of up to four tokens whose x
// rows it stages in LDS as float32. A wave loads its row slice once into
// registers (coalesced: row element 64c + l goes to lane l) and forms each
// token's float32 dot product in the stated order: lane l keeps the partial
// sum of the terms h = 64c + l for c = 0, 1, ... (multiply and add rounded
// separately, contraction disabled), then the halving tree
// p[l] += p[l + off], off = 32 .. 1, with shuffles; the bias is added last.
// The top-k kernel then gives each token one wave: the top-k by repeated
// wave-wide maxima of a 64-bit key (order-preserving float bits, then
// inverted expert ID, so ties go to the lower ID), the softmax weights over
// all E logits and the sigmoid of the shared-gate dot.
#include <algorithm>

#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kRowsPerWg = 8;               // router rows per logits workgroup (one per wave)
constexpr int kLogitThreads = kRowsPerWg * kWave;
constexpr int kMaxTokTile = 4;              // tokens per logits workgroup
constexpr int kSlice = 32;                  // row chunks of 64 held in registers (2048 h)
constexpr int kTopkWaves = 4;               // tokens per top-k workgroup

struct RouteArgs {
  const _Float16* x;
  const float* w;
  const float* bias;
  const float* gate_w;
  int32_t* ids;
  float* wout;
  float* logits;
  float* gate;                              // raw gate dot, then its sigmoid
  int T, H, E, k, flags, tok_tile;
};

// Increasing map float -> uint32 with -0.0 and +0.0 sent to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kLogitThreads) void logits_kernel(RouteArgs a) {
#pragma clang fp contract(off)
  extern __shared__ float xs[];             // [tok_tile][H]
  const int H = a.H, E = a.E;
  const int t0 = blockIdx.y * a.tok_tile;
  const int tt = min(a.tok_tile, a.T - t0);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;

  // x rows of the tile, 8 halves per load
  const int n8 = tt * H / 8;
  const _Float16* xt = a.x + static_cast<size_t>(t0) * H;
  for (int i = threadIdx.x; i < n8; i += kLogitThreads) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 v = *reinterpret_cast<const h8*>(xt + 8 * i);
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[8 * i + j] = static_cast<float>(v[j]);
  }
  __syncthreads();

  const bool want_gate = a.gate_w != nullptr && a.gate != nullptr;
  const int r = blockIdx.x * kRowsPerWg + wave;
  if (r >= E + (want_gate ? 1 : 0)) return;
  const float* wr = r < E ? a.w + static_cast<size_t>(r) * H : a.gate_w;
  const int nc = H / kWave;
  float p[kMaxTokTile];
#pragma unroll
  for (int t = 0; t < kMaxTokTile; ++t) p[t] = 0.0f;
  for (int c0 = 0; c0 < nc; c0 += kSlice) {
    float w[kSlice];
#pragma unroll
    for (int j = 0; j < kSlice; ++j) w[j] = wr[min(c0 + j, nc - 1) * kWave + lane];
#pragma unroll
    for (int t = 0; t < kMaxTokTile; ++t) {
      if (t < tt) {
        const float* xr = xs + t * H + lane;
#pragma unroll
        for (int j = 0; j < kSlice; ++j) {
          if (c0 + j < nc) {
            const float prod = xr[(c0 + j) * kWave] * w[j];
            p[t] = p[t] + prod;
          }
        }
      }
    }
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
#pragma unroll
    for (int t = 0; t < kMaxTokTile; ++t) {
      const float o = __shfl_down(p[t], off, kWave);
      p[t] = p[t] + o;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < kMaxTokTile; ++t) {
      if (t < tt) {
        float v = p[t];
        if (r < E) {
          if (a.bias != nullptr) v = v + a.bias[r];
          a.logits[static_cast<size_t>(t0 + t) * E + r] = v;
        } else {
          a.gate[t0 + t] = v;
        }
      }
    }
  }
}

__global__ __launch_bounds__(kTopkWaves * kWave) void topk_kernel(RouteArgs a) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kTopkWaves + threadIdx.x / kWave;
  if (t >= a.T) return;
  const int E = a.E;
  const float* l = a.logits + static_cast<size_t>(t) * E;

  float lv[kMaxE / kWave];
  uint64_t key[kMaxE / kWave];
#pragma unroll
  for (int i = 0; i < kMaxE / kWave; ++i) {
    const int e = lane + i * kWave;
    lv[i] = e < E ? l[e] : 0.0f;
    key[i] = e < E ? (static_cast<uint64_t>(order_key(lv[i])) << 32) |
                         static_cast<uint32_t>(0xFFFFFFFFu - static_cast<uint32_t>(e))
                   : 0ull;
  }
  int my_sel = 0;
  uint64_t first = 0ull;
  for (int j = 0; j < a.k; ++j) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFull));
    if (j == 0) first = best;
    if (lane == j) my_sel = e;
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; ++i)
      if (lane + i * kWave == e) key[i] = 0ull;
  }

  // softmax over all E logits, evaluated at the selected experts
  const int e_first =
      static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(first & 0xFFFFFFFFull));
  const float mx = l[e_first];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxE / kWave; ++i) {
    const int e = lane + i * kWave;
    if (e < E) s += expf(lv[i] - mx);
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
  if (a.gate != nullptr && a.gate_w != nullptr && lane == 0)
    a.gate[t] = 1.0f / (1.0f + expf(-a.gate[t]));
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
  SMOE_REQUIRE(x && w_router && topk_ids && topk_w && logits, SMOE_EINVAL,
               "route_topk: null pointer (x, w_router, topk_ids, topk_w and logits are required)");
  SMOE_REQUIRE(aligned16(x), SMOE_EINVAL, "route_topk: x must be 16-byte aligned");
  SMOE_REQUIRE(static_cast<long long>(T) * k < (1ll << 24), SMOE_EUNSUPPORTED,
               "route_topk: T*k must be below 2^24");

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
  // tokens per logits workgroup: up to four, x tile within 64 KB of LDS
  a.tok_tile = std::max(1, std::min(kMaxTokTile, 65536 / (H * 4)));
  const int nrows = E + (shared_gate_w != nullptr ? 1 : 0);
  const dim3 grid((nrows + kRowsPerWg - 1) / kRowsPerWg, (T + a.tok_tile - 1) / a.tok_tile);
  const size_t lds = static_cast<size_t>(a.tok_tile) * H * sizeof(float);
  hipStream_t st = as_stream(stream);
  hipLaunchKernelGGL(logits_kernel, grid, dim3(kLogitThreads), lds, st, a);
  smoe_status s = check_launch("route_topk logits");
  if (s != SMOE_OK) return s;
  hipLaunchKernelGGL(topk_kernel, dim3((T + kTopkWaves - 1) / kTopkWaves),
                     dim3(kTopkWaves * kWave), 0, st, a);
  return check_launch("route_topk");
}
