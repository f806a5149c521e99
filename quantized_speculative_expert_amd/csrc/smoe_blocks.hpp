// Device building blocks shared by the routing kernels: the per-token
// top-k of the router, the counting sort of slots by expert and the ELB
// counter update with its top-M ranking. Each exists as a kernel of its own
// (route.hip, align.hip, elb.hip) and, for short windows, all three run
// back to back in one workgroup (route.hip); that block is written for any
// workgroup size.
#pragma once

#include "smoe_internal.hpp"

namespace smoe {

// Workgroup barrier that orders LDS only. The blocks below hand over LDS
// data between threads; their global outputs each go to an address that
// one thread writes once and no thread of the block reads back, so the
// barrier need not wait for the stores to complete (a full __syncthreads
// waits for every store in flight, a memory round trip per barrier).
__device__ __forceinline__ void block_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------------ top-k

// Increasing map float -> uint32 with -0.0 and +0.0 sent to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave: the top-k experts of one token from its E logits `l` and their
// softmax weights over all E logits (renormalised over the k with
// SMOE_ROUTE_RENORM). Each expert gets a 64-bit key (order-preserving float
// bits, then inverted expert ID, so ties go to the lower ID; keys are
// distinct) and its rank is the number of larger keys, counted against the
// wave's keys in `lds_keys` (kMaxE words of LDS per wave); the expert of
// rank j is the j-th pick. Lane j < k returns the j-th expert in *id and
// its weight in *w. `lds_sel` holds kMaxK words of LDS per wave.
template <int NK>  // keys per lane: E <= 64 * NK
__device__ __forceinline__ void wave_topk_n(const float* l, int E, int k, int flags,
                                            uint64_t* lds_keys, int* lds_sel, int* id, float* w) {
  const int lane = lane_id();
  float lv[NK];
  uint64_t key[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lane + i * kWave;
    lv[i] = e < E ? l[e] : 0.0f;
    key[i] = (static_cast<uint64_t>(order_key(lv[i])) << 32) |
             static_cast<uint32_t>(0xFFFFFFFFu - static_cast<uint32_t>(e));
    if (e < E) lds_keys[e] = key[i];
    else if (e < ((E + 7) & ~7)) lds_keys[e] = 0ull;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  int rank[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) rank[i] = 0;
  // keys past E read as zero, which no real key is below
  for (int f0 = 0; f0 < E; f0 += 8) {
    uint64_t kf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kf[j] = lds_keys[f0 + j];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < NK; ++i) rank[i] += kf[j] > key[i] ? 1 : 0;
  }
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lane + i * kWave;
    if (e < E && rank[i] < k) lds_sel[rank[i]] = e;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  // softmax over all E logits, evaluated at the selected experts
  const float mx = l[lds_sel[0]];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lane + i * kWave;
    if (e < E) s += expf(lv[i] - mx);
  }
  s = wave_sum_f(s);
  const int my_sel = lane < k ? lds_sel[lane] : 0;
  float wj = lane < k ? expf(l[my_sel] - mx) / s : 0.0f;
  if (flags & SMOE_ROUTE_RENORM) {
    const float tot = wave_sum_f(wj);
    wj = wj / tot;
  }
  *id = my_sel;
  *w = wj;
  __builtin_amdgcn_wave_barrier();  // the wave's LDS words may be reused after this
}

__device__ __forceinline__ void wave_topk(const float* l, int E, int k, int flags,
                                          uint64_t* lds_keys, int* lds_sel, int* id, float* w) {
  if (E <= kWave)
    wave_topk_n<1>(l, E, k, flags, lds_keys, lds_sel, id, w);
  else if (E <= 2 * kWave)
    wave_topk_n<2>(l, E, k, flags, lds_keys, lds_sel, id, w);
  else
    wave_topk_n<kMaxE / kWave>(l, E, k, flags, lds_keys, lds_sel, id, w);
}

// ------------------------------------------------------------------ align

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;

// LDS of align_block for a workgroup of NT threads.
template <int NT>
struct alignas(16) AlignSmemT {
  int wave_cnt[NT / kWave][kMaxE];   // pass 1 counts, then running counters
  int wave_base[NT / kWave][kMaxE];  // slots of expert e in earlier waves
  int exp_off[kMaxE + 1];
  int act_pos[kMaxE];
  int act_list[kMaxE];               // the active list, -1 past its end
};
using AlignSmem = AlignSmemT<kAlignThreads>;

// One workgroup of NT threads: stable counting sort of the S slots by
// expert. Each wave owns a contiguous run of slots and walks it 64 slots at
// a time. Within a 64-slot chunk, the lanes holding the same expert are
// found with eight ballots (one per bit of the expert ID), and a lane's
// rank among them is the popcount of those lanes below it.
//   pass 1: per-wave, per-expert counts (LDS adds, order-free);
//   scan:   expert counts, exclusive offsets, per-wave bases, active list;
//   pass 2: each wave re-walks its run in order and writes slot s to
//           offsets[e] + base[wave][e] + running[wave][e] + rank, which is
//           its position in (expert, slot) order.
// `ids` may point to global or LDS memory.
template <int NT>
__device__ __forceinline__ void align_block_t(const int32_t* ids, int S, int E, int32_t* counts,
                                              int32_t* offsets, int32_t* sorted_slots,
                                              int32_t* active, int32_t* n_active,
                                              AlignSmemT<NT>& sm) {
  constexpr int kWaves = NT / kWave;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;

  for (int i = threadIdx.x; i < kWaves * kMaxE; i += NT)
    (&sm.wave_cnt[0][0])[i] = 0;
  block_sync_lds();

  // contiguous run of whole 64-slot chunks per wave
  const int nchunks = (S + kWave - 1) / kWave;
  const int per_wave = (nchunks + kWaves - 1) / kWaves;
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
    if (e >= 0 && e < E) atomicAdd(&sm.wave_cnt[wave][e], 1);
  };
#pragma unroll
  for (int j = 0; j < kCached; ++j) count(cached[j]);
  for (int c = c_begin + kCached; c < c_end; ++c) {
    const int s = c * kWave + lane;
    count(s < S ? ids[s] : -1);
  }
  block_sync_lds();

  // per expert: total, per-wave bases (only waves that own slots count)
  const int busy_waves = per_wave > 0 ? min(kWaves, (nchunks + per_wave - 1) / per_wave) : 0;
  for (int e = threadIdx.x; e < E; e += NT) {
    int run = 0;
    for (int w = 0; w < busy_waves; ++w) {
      sm.wave_base[w][e] = run;
      run += sm.wave_cnt[w][e];
    }
    counts[e] = run;
    sm.exp_off[e] = run;  // scanned below
  }
  block_sync_lds();

  // exclusive scan over experts (E <= 256, 4 per lane of wave 0) and the
  // ascending active list
  if (wave == 0) {
    int v[4], a[4];
    int vs = 0, as = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      v[i] = e < E ? sm.exp_off[e] : 0;
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
        sm.exp_off[e] = vrun;
        sm.act_pos[e] = a[i] ? arun : -1;
      }
      vrun += v[i];
      arun += a[i];
    }
    const int total = __shfl(v_incl, kWave - 1, kWave);
    const int nact = __shfl(a_incl, kWave - 1, kWave);
    if (lane == 0) {
      sm.exp_off[E] = total;
      offsets[E] = total;
      n_active[0] = nact;
    }
  }
  block_sync_lds();

  // (each output word written once: the active list is built in LDS first)
  for (int e = threadIdx.x; e < E; e += NT) {
    offsets[e] = sm.exp_off[e];
    sm.act_list[e] = -1;
  }
  block_sync_lds();
  for (int e = threadIdx.x; e < E; e += NT)
    if (sm.act_pos[e] >= 0) sm.act_list[sm.act_pos[e]] = e;
  block_sync_lds();
  for (int e = threadIdx.x; e < E; e += NT) active[e] = sm.act_list[e];
  for (int p = sm.exp_off[E] + threadIdx.x; p < S; p += NT) sorted_slots[p] = -1;

  // pass 2: stable placement; wave_cnt becomes the running count per wave
  for (int i = lane; i < E; i += kWave) sm.wave_cnt[wave][i] = 0;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup", "local");
  auto place = [&](int c, int e) {
    const int s = c * kWave + lane;
    const bool valid = e >= 0 && e < E;
    const uint64_t same = match_key8(valid ? e : 0, valid);
    const int rank = __popcll(same & lanes_below_mask());
    if (valid) {
      const int pos = sm.exp_off[e] + sm.wave_base[wave][e] + sm.wave_cnt[wave][e] + rank;
      sorted_slots[pos] = s;
    }
    // the highest-ranked lane of each group advances its expert's counter
    const bool last = valid && (same >> lane) == 1ull;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup", "local");
    if (last) sm.wave_cnt[wave][e] += rank + 1;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup", "local");
  };
#pragma unroll
  for (int j = 0; j < kCached; ++j)
    if (c_begin + j < c_end) place(c_begin + j, cached[j]);
  for (int c = c_begin + kCached; c < c_end; ++c) {
    const int s = c * kWave + lane;
    place(c, s < S ? ids[s] : -1);
  }
}

__device__ __forceinline__ void align_block(const int32_t* ids, int S, int E, int32_t* counts,
                                            int32_t* offsets, int32_t* sorted_slots,
                                            int32_t* active, int32_t* n_active, AlignSmem& sm) {
  align_block_t<kAlignThreads>(ids, S, E, counts, offsets, sorted_slots, active, n_active, sm);
}

// ------------------------------------------------------------------ ELB

// One workgroup, one layer: adds the histogram of the layer's S routed IDs
// `lid` (when not null) to its counter row `crow` (integer adds, so the
// result does not depend on timing); then, with M > 0, expert e's place is
// the number of experts ahead of it in (count descending, ID ascending)
// order, and experts placed below M write themselves into the plan; then,
// with `clear`, the row is zeroed. hist and row are LDS scratch of kMaxE.
// With PRE, `pre` (LDS) already holds the row as crow had it, read before
// the block wrote anything (a load issued after stores waits for them).
// `lid` is read only with `add` (so one pointer serves every layer).
template <bool PRE = false>
__device__ __forceinline__ void elb_block(int32_t* crow, int E, const int32_t* lid, bool add,
                                          int S, int M, int32_t* plan_ids, int32_t* plan_counts,
                                          int clear, int* hist, int* row,
                                          const int* pre = nullptr) {
  const int nt = blockDim.x;
  for (int e = threadIdx.x; e < E; e += nt) hist[e] = 0;
  block_sync_lds();
  if (add) {
    for (int s = threadIdx.x; s < S; s += nt) {
      const int e = lid[s];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  block_sync_lds();
  for (int e = threadIdx.x; e < E; e += nt) {
    const int v = (PRE ? pre[e] : crow[e]) + hist[e];
    row[e] = v;
    if (hist[e] != 0) crow[e] = v;
  }
  block_sync_lds();
  if (M > 0) {
    // expert e's place counted by kParts consecutive lanes, each over a
    // share of the row, summed with shuffles within the lane group
    constexpr int kParts = 16;
    const int per = (E + kParts - 1) / kParts;
    for (int base = threadIdx.x; base < E * kParts; base += nt) {  // (nt % kParts == 0)
      const int e = base / kParts, part = base % kParts;
      const int c = row[e];
      int place = 0;
      for (int f = part * per; f < min(E, (part + 1) * per); ++f) {
        const int cf = row[f];
        place += (cf > c || (cf == c && f < e)) ? 1 : 0;
      }
#pragma unroll
      for (int off = kParts / 2; off >= 1; off >>= 1) place += __shfl_xor(place, off, kWave);
      if (part == 0 && place < M) {
        plan_ids[place] = e;
        if (plan_counts != nullptr) plan_counts[place] = c;
      }
    }
  }
  if (clear) {
    for (int e = threadIdx.x; e < E; e += nt) crow[e] = 0;
  }
}


// ------------------------------------------------------------------ routing

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

// Top-k, alignment and the ELB update of one layer in one workgroup, for
// windows of at most kFusedMaxSlots slots.
constexpr int kFusedMaxSlots = 512;
constexpr int kFusedMaxLogits = 4096;  // logits staged in LDS up to this many

struct FusedArgs {
  RouteArgs r;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_slots;
  int32_t* active;
  int32_t* n_active;
  int32_t* elb_counts;  // [L][E] or null (no ELB update)
  int32_t* plan_ids;
  int32_t* plan_counts;
  int L, layer, M, elb_clear;
  // Weights that the launch's other workgroups read through the caches
  // while the routing workgroup works (16-byte units; none when pf_n are 0).
  const uint4* pf[3];
  long long pf_n[3];
  int pf_never;  // always zero; its test keeps the loads, which store nothing
};

// Argument checks of smoe_route_topk, filling `a` (route.hip); the one-call
// layer (ffn.hip) runs them before it enqueues anything.
smoe_status route_check(const void* x, const float* w_router, const float* logit_bias, int T,
                        int H, int E, int k, int flags, int32_t* topk_ids, float* topk_w,
                        float* logits, const float* shared_gate_w, float* shared_gate,
                        RouteArgs& a);

// The fused routing call with an optional list of weights that `wgs` more
// workgroups of the routing launch read through the caches while its one
// routing workgroup works (smoe_route_align_elb passes none). The layer
// call lists the shared experts' FP16 weights, which do not depend on the
// routing: the FFN's first items then find them in the Infinity Cache
// instead of waiting on HBM, and HBM is otherwise idle during the routing.
struct RoutePrefetch {
  const void* p[3];
  long long bytes[3];  // multiples of 16
  int wgs;
};
smoe_status route_align_elb(
    const void* x, const float* w_router, const float* logit_bias, int T, int H, int E, int k,
    int flags, int32_t* topk_ids, float* topk_w, float* logits, const float* shared_gate_w,
    float* shared_gate, int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
    int32_t* active_experts, int32_t* n_active, int32_t* elb_counts, int L, int layer, int M,
    int32_t* plan_ids, int32_t* plan_counts, int elb_flags, void* stream,
    const RoutePrefetch* pf);

// (NLG: logits the block can stage, at least T * E, plus T for a staged
// shared gate)
template <int NT, int NLG = kFusedMaxLogits>
struct alignas(16) RouteBlockSmem {
  AlignSmemT<NT> al;
  int ids[kFusedMaxSlots];
  int hist[kMaxE];
  int row[kMaxE];
  int pre[kMaxE];                     // the layer's counter row, read first
  float lg[NLG];
};

// One workgroup of NT threads, after the router logits: wave w takes the
// top-k of tokens w, w + NT/64, ... (the IDs also go to LDS), then
// align_block_t sorts the slots from LDS, then elb_block updates the
// layer's counter row and ranks every layer. The results equal those of the
// three separate kernels. With `staged`, the caller has already put the
// T x E logits in sm.lg, followed by the T raw shared-gate dots (when the
// layer has a gate), and the block reads neither from global memory.
template <int NT, int NLG>
__device__ __forceinline__ void route_align_elb_block(const FusedArgs& f,
                                                      RouteBlockSmem<NT, NLG>& sm,
                                                      bool staged = false) {
  constexpr int kWaves = NT / kWave;
  const RouteArgs& a = f.r;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  // the top-k's per-wave LDS words live in the alignment's scratch, which is
  // not in use yet
  static_assert(sizeof(sm.al.wave_cnt) + sizeof(sm.al.wave_base) >= kWaves * kMaxE * 8,
                "per-wave top-k keys fit the alignment scratch");
  static_assert(sizeof(sm.al.exp_off) >= kWaves * kMaxK * 4, "per-wave picks fit");
  uint64_t* keys = reinterpret_cast<uint64_t*>(&sm.al.wave_cnt[0][0]) + wave * kMaxE;
  int* sel = &sm.al.exp_off[0] + wave * kMaxK;
  // all logits in one round trip when they fit, then the top-k from LDS
  // Global loads first (the logits unless staged, the layer's counter row):
  // any load issued after a store waits for that store's round trip.
  const int n_lg = a.T * a.E;
  const bool lg_in_lds = staged || n_lg <= NLG;
  if (lg_in_lds && !staged)
    for (int i = threadIdx.x; i < n_lg; i += NT) sm.lg[i] = a.logits[i];
  if (f.elb_counts != nullptr)
    for (int e = threadIdx.x; e < a.E; e += NT)
      sm.pre[e] = f.elb_counts[static_cast<size_t>(f.layer) * a.E + e];
  block_sync_lds();
  const bool want_gate = a.gate != nullptr && a.gate_w != nullptr;
  for (int t = wave; t < a.T; t += kWaves) {
    int id;
    float w;
    float raw = 0.0f;
    if (want_gate && lane == 0) raw = staged ? sm.lg[n_lg + t] : a.gate[t];
    // (two calls, so that each reads through its own address space)
    if (lg_in_lds)
      wave_topk(sm.lg + t * a.E, a.E, a.k, a.flags, keys, sel, &id, &w);
    else
      wave_topk(a.logits + static_cast<size_t>(t) * a.E, a.E, a.k, a.flags, keys, sel, &id, &w);
    if (lane < a.k) {
      a.ids[static_cast<size_t>(t) * a.k + lane] = id;
      a.wout[static_cast<size_t>(t) * a.k + lane] = w;
      sm.ids[t * a.k + lane] = id;
    }
    if (want_gate && lane == 0) a.gate[t] = 1.0f / (1.0f + expf(-raw));
  }
  block_sync_lds();
  const int S = a.T * a.k;
  align_block_t<NT>(sm.ids, S, a.E, f.counts, f.offsets, f.sorted_slots, f.active, f.n_active,
                    sm.al);
  if (f.elb_counts == nullptr) return;
  for (int l = 0; l < f.L; ++l) {
    block_sync_lds();
    int32_t* crow = f.elb_counts + static_cast<size_t>(l) * a.E;
    int32_t* pid = f.plan_ids + static_cast<size_t>(l) * f.M;
    int32_t* pc = f.plan_counts != nullptr ? f.plan_counts + static_cast<size_t>(l) * f.M : nullptr;
    if (l == f.layer)
      elb_block<true>(crow, a.E, sm.ids, true, S, f.M, pid, pc, f.elb_clear, sm.hist, sm.row,
                      sm.pre);
    else
      elb_block(crow, a.E, sm.ids, false, S, f.M, pid, pc, f.elb_clear, sm.hist, sm.row);
  }
}

}  // namespace smoe
