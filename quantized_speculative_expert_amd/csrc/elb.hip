// smoe_elb_accumulate_topm: ELB activation counter and top-M prefetch plan.
//
// Specter paper, Incremental Routing Pattern Analyzer paragraphs: per layer
// j and expert e, the counter ELB_cnt[j, e] holds how many draft tokens so
// far had e among their top-k experts in layer j; it lives on the GPU. At a
// prefetch checkpoint each layer's experts are ordered by that count, the
// first M (as many as the layer has cache slots) make up the plan, and the
// counters go back to zero when drafting ends. Design notes, "Predictive I/O
// Orchestrator" (the pattern analyzer).
//
// One workgroup per layer. Accumulation: an LDS histogram of the layer's
// T*k IDs (integer adds, order-free) added to the counter row, which only
// this workgroup touches. Ranking: expert e's place is the number of
// experts ahead of it in (count descending, ID ascending) order, found by
// one pass over the LDS copy of the row; experts placed below M write
// themselves into the plan. Integer only, so the result is exact and
// independent of thread timing.
#include "smoe_blocks.hpp"

namespace smoe {
namespace {

constexpr int kElbThreads = 256;

__global__ __launch_bounds__(kElbThreads) void elb_kernel(
    int32_t* __restrict__ cnt, int E, const int32_t* __restrict__ ids, int layer_begin,
    int n_layers, int S, int M, int32_t* __restrict__ plan_ids,
    int32_t* __restrict__ plan_counts, int clear) {
  __shared__ int hist[kMaxE];
  __shared__ int row[kMaxE];
  const int l = blockIdx.x;
  const int i = l - layer_begin;
  const int32_t* lid =
      (ids != nullptr && i >= 0 && i < n_layers) ? ids + static_cast<size_t>(i) * S : nullptr;
  elb_block(cnt + static_cast<size_t>(l) * E, E, lid, lid != nullptr, S, M,
            plan_ids + static_cast<size_t>(l) * M,
            plan_counts != nullptr ? plan_counts + static_cast<size_t>(l) * M : nullptr, clear,
            hist, row);
}

}  // namespace
}  // namespace smoe

using namespace smoe;

namespace smoe {

smoe_status elb_check(const int32_t* elb_counts, int L, int E, const int32_t* topk_ids,
                      int layer_begin, int n_layers, int T, int k, int M, const int32_t* plan_ids,
                      int flags) {
  SMOE_REQUIRE(L > 0 && E > 0 && M >= 0, SMOE_EINVAL,
               "elb_accumulate_topm: need L > 0, E > 0, M >= 0 (L=%d E=%d M=%d)", L, E, M);
  SMOE_REQUIRE(E <= kMaxE, SMOE_EUNSUPPORTED, "elb_accumulate_topm: E must be <= 256 (E=%d)", E);
  SMOE_REQUIRE(M <= E, SMOE_EINVAL, "elb_accumulate_topm: M must be <= E (M=%d E=%d)", M, E);
  SMOE_REQUIRE((flags & ~SMOE_ELB_CLEAR_AFTER) == 0, SMOE_EINVAL,
               "elb_accumulate_topm: unknown flags %d", flags);
  SMOE_REQUIRE(elb_counts != nullptr, SMOE_EINVAL, "elb_accumulate_topm: null counter");
  SMOE_REQUIRE(M == 0 || plan_ids != nullptr, SMOE_EINVAL, "elb_accumulate_topm: null plan_ids");
  if (topk_ids != nullptr) {
    SMOE_REQUIRE(T >= 0 && k > 0 && n_layers >= 0, SMOE_EINVAL,
                 "elb_accumulate_topm: need T >= 0, k > 0, n_layers >= 0");
    SMOE_REQUIRE(k <= kMaxK, SMOE_EUNSUPPORTED, "elb_accumulate_topm: k must be <= 8");
    SMOE_REQUIRE(layer_begin >= 0 && layer_begin + n_layers <= L, SMOE_EINVAL,
                 "elb_accumulate_topm: layers [%d, %d) outside [0, %d)", layer_begin,
                 layer_begin + n_layers, L);
    SMOE_REQUIRE(static_cast<long long>(T) * k < (1ll << 24), SMOE_EUNSUPPORTED,
                 "elb_accumulate_topm: T*k must be below 2^24");
  }
  return SMOE_OK;
}

}  // namespace smoe

extern "C" smoe_status smoe_elb_accumulate_topm(int32_t* elb_counts, int L, int E,
                                                const int32_t* topk_ids, int layer_begin,
                                                int n_layers, int T, int k, int M,
                                                int32_t* plan_ids, int32_t* plan_counts,
                                                int flags, void* stream) {
  clear_error();
  const smoe_status st =
      elb_check(elb_counts, L, E, topk_ids, layer_begin, n_layers, T, k, M, plan_ids, flags);
  if (st != SMOE_OK) return st;
  const int S = topk_ids != nullptr ? T * k : 0;
  hipLaunchKernelGGL(elb_kernel, dim3(L), dim3(kElbThreads), 0, as_stream(stream), elb_counts, E,
                     topk_ids, layer_begin, topk_ids ? n_layers : 0, S, M, plan_ids, plan_counts,
                     (flags & SMOE_ELB_CLEAR_AFTER) ? 1 : 0);
  return check_launch("elb_accumulate_topm");
}
