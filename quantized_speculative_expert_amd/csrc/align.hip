// smoe_align_by_expert: stable counting sort of routing slots by expert.
//
// Specter paper, fused multi-expert draft kernel paragraph (routed tokens
// are first gathered by expert assignment) and expert-wise verification
// paragraph (tokens of each expert packed into a contiguous sub-batch);
// design notes, "Streamlined Execution Engine" (kernels align token groups).
//
// One workgroup of 16 waves runs align_block (smoe_blocks.hpp).
#include "smoe_blocks.hpp"

namespace smoe {
namespace {

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int S, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ AlignSmem sm;
  align_block(ids, S, E, counts, offsets, sorted_slots, active, n_active, sm);
}

}  // namespace
}  // namespace smoe

using namespace smoe;

namespace smoe {

smoe_status align_check(const int32_t* topk_ids, int T, int k, int E, const int32_t* expert_counts,
                        const int32_t* expert_offsets, const int32_t* sorted_slots,
                        const int32_t* active_experts, const int32_t* n_active) {
  SMOE_REQUIRE(T >= 0 && k > 0 && E > 0, SMOE_EINVAL,
               "align_by_expert: need T >= 0, k > 0, E > 0 (T=%d k=%d E=%d)", T, k, E);
  SMOE_REQUIRE(E <= kMaxE && k <= kMaxK, SMOE_EUNSUPPORTED,
               "align_by_expert: need E <= 256 and k <= 8 (E=%d k=%d)", E, k);
  SMOE_REQUIRE(static_cast<long long>(T) * k < (1ll << 24), SMOE_EUNSUPPORTED,
               "align_by_expert: T*k must be below 2^24");
  SMOE_REQUIRE(expert_counts && expert_offsets && active_experts && n_active, SMOE_EINVAL,
               "align_by_expert: null pointer");
  SMOE_REQUIRE(T * k == 0 || (topk_ids && sorted_slots), SMOE_EINVAL,
               "align_by_expert: null pointer");
  return SMOE_OK;
}

}  // namespace smoe

extern "C" smoe_status smoe_align_by_expert(const int32_t* topk_ids, int T, int k, int E,
                                            int32_t* expert_counts, int32_t* expert_offsets,
                                            int32_t* sorted_slots, int32_t* active_experts,
                                            int32_t* n_active, void* stream) {
  clear_error();
  const smoe_status st = align_check(topk_ids, T, k, E, expert_counts, expert_offsets,
                                     sorted_slots, active_experts, n_active);
  if (st != SMOE_OK) return st;
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, as_stream(stream), topk_ids,
                     T * k, E, expert_counts, expert_offsets, sorted_slots, active_experts,
                     n_active);
  return check_launch("align_by_expert");
}
