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

#include "smoe_blocks.hpp"

namespace smoe {
namespace {

constexpr int kRowsPerWg = 8;               // router rows per logits workgroup (one per wave)
constexpr int kLogitThreads = kRowsPerWg * kWave;
constexpr int kMaxTokTile = 4;              // tokens per logits workgroup, at most
constexpr int kLogitWgTarget = 256;         // logits workgroups wanted (about one per CU)
constexpr int kSlice = 32;                  // row chunks of 64 held in registers (2048 h)
constexpr int kTopkWaves = 4;               // tokens per top-k workgroup


// Staged x of a token tile, transposed so that lane l finds its terms
// h = 64c + l at consecutive c: xs[(t * 64 + l) * ncp + c], with the row
// padded to ncp = round_up(H / 64, 4) + 4 floats (16-byte aligned rows,
// conflict-free 16-byte reads across a quarter wave).
__host__ __device__ inline int logits_ncp(int H) { return (H / kWave + 3) / 4 * 4 + 4; }

__global__ __launch_bounds__(kLogitThreads) void logits_kernel(RouteArgs a) {
#pragma clang fp contract(off)
  extern __shared__ __align__(16) float xs[];
  const int H = a.H, E = a.E;
  const int t0 = blockIdx.y * a.tok_tile;
  const int tt = min(a.tok_tile, a.T - t0);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int nc = H / kWave;
  const int ncp = logits_ncp(H);

  const bool want_gate = a.gate_w != nullptr && a.gate != nullptr;
  const int r = blockIdx.x * kRowsPerWg + wave;
  const bool live = r < E + (want_gate ? 1 : 0);
  // (a wave past the last row reads row 0 and writes nothing)
  const float* wr = !live ? a.w : r < E ? a.w + static_cast<size_t>(r) * H : a.gate_w;
  // the row's first slice is requested before x is staged: the two round
  // trips overlap
  float w[kSlice];
#pragma unroll
  for (int j = 0; j < kSlice; ++j) w[j] = wr[min(j, nc - 1) * kWave + lane];

  // x rows of the tile, 8 halves per load, stored transposed
  const int n8 = tt * H / 8;
  const _Float16* xt = a.x + static_cast<size_t>(t0) * H;
  for (int i = threadIdx.x; i < n8; i += kLogitThreads) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 v = *reinterpret_cast<const h8*>(xt + 8 * i);
    const int t = i / (H / 8);
    const int h = 8 * i - t * H;
    const int c = h / kWave, l = h % kWave;
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[(t * kWave + l + j) * ncp + c] = static_cast<float>(v[j]);
  }
  __syncthreads();
  if (!live) return;

  float p[kMaxTokTile];
#pragma unroll
  for (int t = 0; t < kMaxTokTile; ++t) p[t] = 0.0f;
  for (int c0 = 0; c0 < nc; c0 += kSlice) {
    if (c0 > 0) {
#pragma unroll
      for (int j = 0; j < kSlice; ++j) w[j] = wr[min(c0 + j, nc - 1) * kWave + lane];
    }
#pragma unroll
    for (int t = 0; t < kMaxTokTile; ++t) {
      if (t < tt) {
        const float* xr = xs + (t * kWave + lane) * ncp + c0;
#pragma unroll
        for (int j4 = 0; j4 < kSlice; j4 += 4) {
          if (c0 + j4 >= nc) break;  // (reads stay within the padded row)
          const float4 xv = *reinterpret_cast<const float4*>(xr + j4);
          const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (c0 + j4 + q < nc) {
              const float prod = xa[q] * w[j4 + q];
              p[t] = p[t] + prod;
            }
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
  __shared__ uint64_t keys[kTopkWaves][kMaxE];
  __shared__ int sel[kTopkWaves][kMaxK];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kTopkWaves + wave;
  if (t >= a.T) return;
  int id;
  float w;
  wave_topk(a.logits + static_cast<size_t>(t) * a.E, a.E, a.k, a.flags, keys[wave], sel[wave],
            &id, &w);
  if (lane < a.k) {
    a.ids[static_cast<size_t>(t) * a.k + lane] = id;
    a.wout[static_cast<size_t>(t) * a.k + lane] = w;
  }
  if (a.gate != nullptr && a.gate_w != nullptr && lane == 0)
    a.gate[t] = 1.0f / (1.0f + expf(-a.gate[t]));
}

// Top-k, alignment and the ELB update of one layer in one workgroup of
// kAlignThreads (smoe_blocks.hpp), for windows of at most kFusedMaxSlots
// slots. The results equal those of the three separate kernels. Workgroups
// past the first only read the prefetch list.
// A prefetch workgroup (blockIdx.x >= 1): 16-byte loads strided over the
// listed weights, eight in flight per lane; the values are folded into one
// word that is stored only under a flag that is never set.
__device__ __forceinline__ void prefetch_block(const FusedArgs& f) {
  const long long stride = static_cast<long long>(gridDim.x - 1) * kAlignThreads;
  const long long first = static_cast<long long>(blockIdx.x - 1) * kAlignThreads + threadIdx.x;
  uint32_t acc = 0;
  for (int r = 0; r < 3; ++r) {
    const uint4* p = f.pf[r];
    const long long n = f.pf_n[r];
    long long u = first;
    for (; u + 7 * stride < n; u += 8 * stride) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p[u + j * stride];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].w;
    }
    for (; u < n; u += stride) acc ^= p[u].x;
  }
  if (f.pf_never) f.counts[0] = static_cast<int32_t>(acc);
}

__global__ __launch_bounds__(kAlignThreads) void topk_align_elb_kernel(FusedArgs f) {
  __shared__ RouteBlockSmem<kAlignThreads> sm;
  if (blockIdx.x > 0) {
    prefetch_block(f);
    return;
  }
  route_align_elb_block(f, sm);
}

}  // namespace
}  // namespace smoe

using namespace smoe;

namespace smoe {

smoe_status route_check(const void* x, const float* w_router, const float* logit_bias, int T,
                        int H, int E, int k, int flags, int32_t* topk_ids, float* topk_w,
                        float* logits, const float* shared_gate_w, float* shared_gate,
                        RouteArgs& a) {
  SMOE_REQUIRE(T >= 0 && H > 0 && E > 0 && k > 0, SMOE_EINVAL,
               "route_topk: need T >= 0, H > 0, E > 0, k > 0 (T=%d H=%d E=%d k=%d)", T, H, E, k);
  SMOE_REQUIRE(E <= kMaxE && k <= kMaxK && k <= E, SMOE_EUNSUPPORTED,
               "route_topk: need E <= 256 and k <= min(8, E) (E=%d k=%d)", E, k);
  SMOE_REQUIRE(H % 128 == 0 && H <= 8192, SMOE_EUNSUPPORTED,
               "route_topk: H must be a multiple of 128 and at most 8192 (H=%d)", H);
  SMOE_REQUIRE((flags & ~SMOE_ROUTE_RENORM) == 0, SMOE_EINVAL, "route_topk: unknown flags %d", flags);
  SMOE_REQUIRE((shared_gate_w == nullptr) == (shared_gate == nullptr), SMOE_EINVAL,
               "route_topk: shared_gate_w and shared_gate must both be set or both NULL");
  if (T > 0) {
    SMOE_REQUIRE(x && w_router && topk_ids && topk_w && logits, SMOE_EINVAL,
                 "route_topk: null pointer (x, w_router, topk_ids, topk_w and logits are "
                 "required)");
    SMOE_REQUIRE(aligned16(x), SMOE_EINVAL, "route_topk: x must be 16-byte aligned");
    SMOE_REQUIRE(static_cast<long long>(T) * k < (1ll << 24), SMOE_EUNSUPPORTED,
                 "route_topk: T*k must be below 2^24");
  }
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
  // Tokens per logits workgroup: up to four, the staged x tile within 64 KB
  // of LDS, and no more than keeps about one workgroup per CU. A workgroup
  // pulls its 8 router rows through one CU, whose outstanding misses bound
  // the kernel at short windows; more, smaller tiles spread the rows over
  // more CUs (the rows are re-read per tile from the caches). At T = 17
  // tiles of one token made the layer about 2 us faster than tiles of four.
  const int row_groups = (E + 1 + kRowsPerWg - 1) / kRowsPerWg;
  const long long by_grid = static_cast<long long>(T) * row_groups / kLogitWgTarget;
  a.tok_tile = static_cast<int>(std::max(1ll, std::min<long long>(
      std::min(kMaxTokTile, 65536 / (kWave * logits_ncp(H) * 4)), by_grid)));
  return SMOE_OK;
}

namespace {

smoe_status launch_logits(const RouteArgs& a, hipStream_t st) {
  const int nrows = a.E + (a.gate_w != nullptr ? 1 : 0);
  const dim3 grid((nrows + kRowsPerWg - 1) / kRowsPerWg, (a.T + a.tok_tile - 1) / a.tok_tile);
  const size_t lds = static_cast<size_t>(a.tok_tile) * kWave * logits_ncp(a.H) * sizeof(float);
  hipLaunchKernelGGL(logits_kernel, grid, dim3(kLogitThreads), lds, st, a);
  return check_launch("route_topk logits");
}

}  // namespace
}  // namespace smoe

extern "C" smoe_status smoe_route_topk(const void* x, const float* w_router,
                                       const float* logit_bias, int T, int H, int E, int k,
                                       int flags, int32_t* topk_ids, float* topk_w,
                                       float* logits, const float* shared_gate_w,
                                       float* shared_gate, void* stream) {
  clear_error();
  RouteArgs a;
  smoe_status s = route_check(x, w_router, logit_bias, T, H, E, k, flags, topk_ids, topk_w,
                              logits, shared_gate_w, shared_gate, a);
  if (s != SMOE_OK || T == 0) return s;
  hipStream_t st = as_stream(stream);
  s = launch_logits(a, st);
  if (s != SMOE_OK) return s;
  hipLaunchKernelGGL(topk_kernel, dim3((T + kTopkWaves - 1) / kTopkWaves),
                     dim3(kTopkWaves * kWave), 0, st, a);
  return check_launch("route_topk");
}

namespace smoe {
smoe_status route_align_elb(
    const void* x, const float* w_router, const float* logit_bias, int T, int H, int E, int k,
    int flags, int32_t* topk_ids, float* topk_w, float* logits, const float* shared_gate_w,
    float* shared_gate, int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
    int32_t* active_experts, int32_t* n_active, int32_t* elb_counts, int L, int layer, int M,
    int32_t* plan_ids, int32_t* plan_counts, int elb_flags, void* stream,
    const RoutePrefetch* pf) {
  RouteArgs a;
  smoe_status s = route_check(x, w_router, logit_bias, T, H, E, k, flags, topk_ids, topk_w,
                              logits, shared_gate_w, shared_gate, a);
  if (s != SMOE_OK) return s;
  s = align_check(topk_ids, T, k, E, expert_counts, expert_offsets, sorted_slots,
                  active_experts, n_active);
  if (s != SMOE_OK) return s;
  if (elb_counts != nullptr) {
    s = elb_check(elb_counts, L, E, topk_ids, layer, 1, T, k, M, plan_ids, elb_flags);
    if (s != SMOE_OK) return s;
  }
  if (T == 0 || T * k > kFusedMaxSlots) {  // the three calls one after the other
    s = smoe_route_topk(x, w_router, logit_bias, T, H, E, k, flags, topk_ids, topk_w, logits,
                        shared_gate_w, shared_gate, stream);
    if (s == SMOE_OK)
      s = smoe_align_by_expert(topk_ids, T, k, E, expert_counts, expert_offsets, sorted_slots,
                               active_experts, n_active, stream);
    if (s == SMOE_OK && elb_counts != nullptr)
      s = smoe_elb_accumulate_topm(elb_counts, L, E, topk_ids, layer, 1, T, k, M, plan_ids,
                                   plan_counts, elb_flags, stream);
    return s;
  }
  hipStream_t st = as_stream(stream);
  s = launch_logits(a, st);
  if (s != SMOE_OK) return s;
  FusedArgs f;
  f.r = a;
  f.counts = expert_counts;
  f.offsets = expert_offsets;
  f.sorted_slots = sorted_slots;
  f.active = active_experts;
  f.n_active = n_active;
  f.elb_counts = elb_counts;
  f.plan_ids = plan_ids;
  f.plan_counts = plan_counts;
  f.L = L;
  f.layer = layer;
  f.M = elb_counts != nullptr ? M : 0;
  f.elb_clear = (elb_flags & SMOE_ELB_CLEAR_AFTER) ? 1 : 0;
  f.pf_never = 0;
  int grid = 1;
  for (int r = 0; r < 3; ++r) {
    const bool on = pf != nullptr && pf->wgs > 0 && pf->p[r] != nullptr;
    f.pf[r] = on ? static_cast<const uint4*>(pf->p[r]) : nullptr;
    f.pf_n[r] = on ? pf->bytes[r] / 16 : 0;
    if (f.pf_n[r] > 0) grid = 1 + pf->wgs;
  }
  hipLaunchKernelGGL(topk_align_elb_kernel, dim3(grid), dim3(kAlignThreads), 0, st, f);
  return check_launch("route_align_elb");
}
}  // namespace smoe

extern "C" smoe_status smoe_route_align_elb(
    const void* x, const float* w_router, const float* logit_bias, int T, int H, int E, int k,
    int flags, int32_t* topk_ids, float* topk_w, float* logits, const float* shared_gate_w,
    float* shared_gate, int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
    int32_t* active_experts, int32_t* n_active, int32_t* elb_counts, int L, int layer, int M,
    int32_t* plan_ids, int32_t* plan_counts, int elb_flags, void* stream) {
  clear_error();
  return route_align_elb(x, w_router, logit_bias, T, H, E, k, flags, topk_ids, topk_w, logits,
                         shared_gate_w, shared_gate, expert_counts, expert_offsets,
                         sorted_slots, active_experts, n_active, elb_counts, L, layer, M,
                         plan_ids, plan_counts, elb_flags, stream, nullptr);
}
