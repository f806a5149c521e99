// smoe_align_by_expert: stable counting sort of routing slots by expert.
//
// Specter paper, fused multi-expert draft kernel paragraph (routed tokens
// are first gathered by expert assignment) and expert-wise verification
// paragraph (tokens of each expert packed into a contiguous sub-batch);
// design notes, "Streamlined Execution Engine" (kernels align token groups).
//
// One workgroup of 16 waves. Each wave owns a contiguous run of slots and
// walks it 64 slots at a time. Within a 64-slot chunk, the lanes holding the
// same expert are found with eight ballots (one per bit of the expert ID),
// and a lane's rank among them is the popcount of those lanes below it.
//   pass 1: per-wave, per-expert counts (LDS adds, order-free);
//   scan:   expert counts, exclusive offsets, per-wave bases, active list;
//   pass 2: each wave re-walks its run in order and writes slot s to
//           offsets[e] + base[wave][e] + running[wave][e] + rank, which is
//           its position in (expert, slot) order.
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int S, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ int wave_cnt[kAlignWaves][kMaxE];   // pass 1 counts, then running counters
  __shared__ int wave_base[kAlignWaves][kMaxE];  // slots of expert e in earlier waves
  __shared__ int exp_off[kMaxE + 1];
  __shared__ int act_pos[kMaxE];

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;

  for (int i = threadIdx.x; i < kAlignWaves * kMaxE; i += kAlignThreads)
    (&wave_cnt[0][0])[i] = 0;
  __syncthreads();

  // contiguous run of whole 64-slot chunks per wave
  const int nchunks = (S + kWave - 1) / kWave;
  const int per_wave = (nchunks + kAlignWaves - 1) / kAlignWaves;
  const int c_begin = wave * per_wave;
  const int c_end = min(nchunks, c_begin + per_wave);

  // the first kCached chunks of a wave's run stay in registers for pass 2
  constexpr int kCached = 4;
  int cached[kCached];
#pragma unroll
  for (int j = 0; j < kCached; ++j) {
    const int s = (c_begin + j) * kWave + lane;
    cached[j] = (c_begin + j < c_end && s < S) ? ids[s] : -1;
  }

  // pass 1: counts per (wave, expert)
  auto count = [&](int e) {
    if (e >= 0 && e < E) atomicAdd(&wave_cnt[wave][e], 1);
  };
#pragma unroll
  for (int j = 0; j < kCached; ++j) count(cached[j]);
  for (int c = c_begin + kCached; c < c_end; ++c) {
    const int s = c * kWave + lane;
    count(s < S ? ids[s] : -1);
  }
  __syncthreads();

  // per expert: total, per-wave bases (only waves that own slots count)
  const int busy_waves = per_wave > 0 ? min(kAlignWaves, (nchunks + per_wave - 1) / per_wave) : 0;
  for (int e = threadIdx.x; e < E; e += kAlignThreads) {
    int run = 0;
    for (int w = 0; w < busy_waves; ++w) {
      wave_base[w][e] = run;
      run += wave_cnt[w][e];
    }
    counts[e] = run;
    exp_off[e] = run;  // scanned below
  }
  __syncthreads();

  // exclusive scan over experts (E <= 256, 4 per lane of wave 0) and the
  // ascending active list
  if (wave == 0) {
    int v[4], a[4];
    int vs = 0, as = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      v[i] = e < E ? exp_off[e] : 0;
      a[i] = (e < E && v[i] > 0) ? 1 : 0;
      vs += v[i];
      as += a[i];
    }
    const int v_incl = wave_inclusive_scan(vs);
    const int a_incl = wave_inclusive_scan(as);
    int vrun = v_incl - vs, arun = a_incl - as;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      if (e < E) {
        exp_off[e] = vrun;
        act_pos[e] = a[i] ? arun : -1;
      }
      vrun += v[i];
      arun += a[i];
    }
    const int total = __shfl(v_incl, kWave - 1, kWave);
    const int nact = __shfl(a_incl, kWave - 1, kWave);
    if (lane == 0) {
      exp_off[E] = total;
      offsets[E] = total;
      n_active[0] = nact;
    }
  }
  __syncthreads();

  for (int e = threadIdx.x; e < E; e += kAlignThreads) {
    offsets[e] = exp_off[e];
    active[e] = -1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kAlignThreads)
    if (act_pos[e] >= 0) active[act_pos[e]] = e;
  for (int p = exp_off[E] + threadIdx.x; p < S; p += kAlignThreads) sorted_slots[p] = -1;

  // pass 2: stable placement; wave_cnt becomes the running count per wave
  for (int i = lane; i < E; i += kWave) wave_cnt[wave][i] = 0;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  auto place = [&](int c, int e) {
    const int s = c * kWave + lane;
    const bool valid = e >= 0 && e < E;
    const uint64_t same = match_key8(valid ? e : 0, valid);
    const int rank = __popcll(same & lanes_below_mask());
    if (valid) {
      const int pos = exp_off[e] + wave_base[wave][e] + wave_cnt[wave][e] + rank;
      sorted_slots[pos] = s;
    }
    // the highest-ranked lane of each group advances its expert's counter
    const bool last = valid && (same >> lane) == 1ull;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    if (last) wave_cnt[wave][e] += rank + 1;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  };
#pragma unroll
  for (int j = 0; j < kCached; ++j)
    if (c_begin + j < c_end) place(c_begin + j, cached[j]);
  for (int c = c_begin + kCached; c < c_end; ++c) {
    const int s = c * kWave + lane;
    place(c, s < S ? ids[s] : -1);
  }
}

}  // namespace
}  // namespace smoe

using namespace smoe;

extern "C" smoe_status smoe_align_by_expert(const int32_t* topk_ids, int T, int k, int E,
                                            int32_t* expert_counts, int32_t* expert_offsets,
                                            int32_t* sorted_slots, int32_t* active_experts,
                                            int32_t* n_active, void* stream) {
  clear_error();
  SMOE_REQUIRE(T >= 0 && k > 0 && E > 0, SMOE_EINVAL,
               "align_by_expert: need T >= 0, k > 0, E > 0 (T=%d k=%d E=%d)", T, k, E);
  SMOE_REQUIRE(E <= kMaxE && k <= kMaxK, SMOE_EUNSUPPORTED,
               "align_by_expert: need E <= 256 and k <= 8 (E=%d k=%d)", E, k);
  SMOE_REQUIRE(static_cast<long long>(T) * k < (1ll << 24), SMOE_EUNSUPPORTED,
               "align_by_expert: T*k must be below 2^24");
  SMOE_REQUIRE(expert_counts && expert_offsets && active_experts && n_active, SMOE_EINVAL,
               "align_by_expert: null pointer");
  const int S = T * k;
  SMOE_REQUIRE(S == 0 || (topk_ids && sorted_slots), SMOE_EINVAL, "align_by_expert: null pointer");
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, as_stream(stream), topk_ids, S,
                     E, expert_counts, expert_offsets, sorted_slots, active_experts, n_active);
  return check_launch("align_by_expert");
}
