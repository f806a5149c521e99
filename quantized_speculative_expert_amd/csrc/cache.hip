// Expert cache of the verification pass and the ELB-driven prefetch planner:
// the host runtime around the expert FFN when the FP16 target experts live
// in host memory and a per-layer pool of device slots caches them.
//
// Specter paper, Layer-Aware Prefetch Planner paragraphs (Cold Start,
// Prefetch Overlap and Final Cleanup; at each chunk boundary the top-M
// ranking of the activation counters selects experts, the ones not cached
// form the next host-to-device batch, and the next boundary is placed so the
// chunk's draft compute covers that batch's transfer time), Verification
// Expert Cache Residency Manager paragraph (hits to the compute queue first,
// misses to the I/O queue and then to the compute queue as they land, slots
// protected until their expert's tokens are done, loaded experts not
// replaced before use), cache-aware execution schedule paragraph (the
// resident expert's sub-batch runs while the missing one is copied) and
// Overlap-Oriented Parallelism Optimizer paragraph (separate compute and I/O
// streams, events for expert readiness and safe slot reuse, pinned host
// memory with asynchronous copies). Design page, "Predictive I/O
// Orchestrator" (expert_cache: resident experts, replacement order, slot
// ownership; residency as a per-layer slot budget).
//
// Decisions are taken on the host from small per-slot state: which expert a
// slot holds, the clock value of its last use (replacement is least recently
// used, ties to the lower slot), and whether the current window's predictions
// claimed it. With device memory attached, the same calls enqueue the copies
// (hipMemcpyAsync on the I/O stream) and the expert FFN launches (on the
// compute stream), ordered by two events per slot: `ready` (the last copy into
// the slot is done) and `released` (the last computation that read it is
// done). Nothing here waits on the host.
#include <algorithm>
#include <cmath>
#include <vector>

#include "smoe_internal.hpp"

struct smoe_expert_cache {
  int L = 0, E = 0, M = 0;
  size_t expert_bytes = 0;
  uint8_t* pool = nullptr;            // device [L][M][expert_bytes], or null
  const uint8_t* host = nullptr;      // host [L][E][expert_bytes], or null
  std::vector<int32_t> held;          // [L][M] expert in the slot, -1 empty
  std::vector<int32_t> where;         // [L][E] slot of the expert, -1 not cached
  std::vector<int64_t> used;          // [L][M] clock of the last use (0 never)
  std::vector<uint8_t> claim;         // [L][M] claimed by this window's predictions
  int64_t clock = 0;
  int device = -1;
  std::vector<hipEvent_t> ready, released;     // [L][M]
  std::vector<uint8_t> ready_on, released_on;  // recorded at least once
};

namespace smoe {
namespace {

using Cache = smoe_expert_cache;

bool device_mode(const Cache* c) { return c->pool != nullptr; }

// Slots a new expert of layer l may take, in the order it takes them: empty
// slots by index, then occupied ones by (last use, index); `skip` marks slots
// it may not take.
void victim_order(const Cache* c, int l, const std::vector<uint8_t>& skip,
                  std::vector<int>& out) {
  out.clear();
  std::vector<int> occupied;
  for (int s = 0; s < c->M; ++s) {
    if (skip[s]) continue;
    if (c->held[l * c->M + s] < 0) out.push_back(s);
    else occupied.push_back(s);
  }
  std::stable_sort(occupied.begin(), occupied.end(), [&](int a, int b) {
    return c->used[l * c->M + a] < c->used[l * c->M + b];
  });
  out.insert(out.end(), occupied.begin(), occupied.end());
}

void place(Cache* c, int l, int s, int e) {
  const int old = c->held[l * c->M + s];
  if (old >= 0) c->where[l * c->E + old] = -1;
  c->held[l * c->M + s] = e;
  if (e >= 0) c->where[l * c->E + e] = s;
}

smoe_status hip_fail(const char* who, const char* what, hipError_t err) {
  set_error("%s: %s failed: %s", who, what, hipGetErrorString(err));
  return SMOE_EHIP;
}

// Copy expert e of layer l into slot s on `io` after the slot's last reader.
smoe_status enqueue_load(Cache* c, int l, int e, int s, hipStream_t io, const char* who) {
  const size_t i = static_cast<size_t>(l) * c->M + s;
  hipError_t err;
  if (c->released_on[i] && (err = hipStreamWaitEvent(io, c->released[i], 0)) != hipSuccess)
    return hip_fail(who, "hipStreamWaitEvent", err);
  err = hipMemcpyAsync(c->pool + i * c->expert_bytes,
                       c->host + (static_cast<size_t>(l) * c->E + e) * c->expert_bytes,
                       c->expert_bytes, hipMemcpyHostToDevice, io);
  if (err != hipSuccess) return hip_fail(who, "hipMemcpyAsync", err);
  if ((err = hipEventRecord(c->ready[i], io)) != hipSuccess)
    return hip_fail(who, "hipEventRecord", err);
  c->ready_on[i] = 1;
  return SMOE_OK;
}

smoe_status check_cache(const Cache* c, const char* who) {
  SMOE_REQUIRE(c != nullptr, SMOE_EINVAL, "%s: null cache", who);
  return SMOE_OK;
}

// One entry of a verification schedule.
struct Step {
  int expert, slot, kind, evicted, wait;
};
constexpr int kHit = 0, kMiss = 1;

// The verification decisions for layer l (commits them to the state).
smoe_status verify_decide(Cache* c, int l, const int32_t* counts, std::vector<Step>& steps,
                          const char* who) {
  steps.clear();
  std::vector<int> hits, misses;
  for (int e = 0; e < c->E; ++e) {
    if (counts[e] <= 0) continue;
    (c->where[l * c->E + e] >= 0 ? hits : misses).push_back(e);
  }
  SMOE_REQUIRE(misses.empty() || c->M > 0, SMOE_EINVAL, "%s: no cache slots for the misses",
               who);
  std::vector<uint8_t> prot(c->M, 0);
  std::vector<int> hit_slots;
  for (int e : hits) {
    prot[c->where[l * c->E + e]] = 1;
    hit_slots.push_back(c->where[l * c->E + e]);
  }
  std::vector<int> free_order;
  victim_order(c, l, prot, free_order);
  // slots that finished computations hand back, in the order they finish
  std::sort(hit_slots.begin(), hit_slots.end());
  std::vector<std::pair<int, int>> handed;  // (slot, group that releases it)
  for (int s : hit_slots) handed.emplace_back(s, 0);
  size_t next_free = 0, next_handed = 0;
  if (!hits.empty()) {
    const int64_t now = ++c->clock;
    for (int e : hits) {
      const int s = c->where[l * c->E + e];
      c->used[l * c->M + s] = now;
      steps.push_back({e, s, kHit, e, -1});
    }
  }
  for (size_t j = 0; j < misses.size(); ++j) {
    int s, wait;
    if (next_free < free_order.size()) {
      s = free_order[next_free++];
      wait = -1;
    } else {
      s = handed[next_handed].first;
      wait = handed[next_handed].second;
      ++next_handed;
    }
    const int e = misses[j];
    steps.push_back({e, s, kMiss, c->held[l * c->M + s], wait});
    place(c, l, s, e);
    c->used[l * c->M + s] = ++c->clock;
    handed.emplace_back(s, 1 + static_cast<int>(j));
  }
  return SMOE_OK;
}

}  // namespace
}  // namespace smoe

using namespace smoe;

extern "C" smoe_status smoe_cache_create(int L, int E, int M, size_t expert_bytes, void* pool,
                                         const void* host_experts, smoe_expert_cache** cache) {
  clear_error();
  const char* who = "cache_create";
  SMOE_REQUIRE(cache != nullptr, SMOE_EINVAL, "%s: null output pointer", who);
  *cache = nullptr;
  SMOE_REQUIRE(L > 0 && E > 0 && M >= 0 && E <= kMaxE, SMOE_EINVAL,
               "%s: need L > 0, 0 < E <= 256 and M >= 0 (L=%d E=%d M=%d)", who, L, E, M);
  SMOE_REQUIRE((pool == nullptr) == (host_experts == nullptr), SMOE_EINVAL,
               "%s: pool and host_experts are both given (copies) or both null (decisions "
               "only)", who);
  SMOE_REQUIRE(pool == nullptr || (expert_bytes > 0 && expert_bytes % 16 == 0), SMOE_EINVAL,
               "%s: expert_bytes must be a positive multiple of 16 (got %zu)", who,
               expert_bytes);
  Cache* c = new Cache();
  c->L = L;
  c->E = E;
  c->M = M;
  c->expert_bytes = expert_bytes;
  c->pool = static_cast<uint8_t*>(pool);
  c->host = static_cast<const uint8_t*>(host_experts);
  c->held.assign(static_cast<size_t>(L) * M, -1);
  c->where.assign(static_cast<size_t>(L) * E, -1);
  c->used.assign(static_cast<size_t>(L) * M, 0);
  c->claim.assign(static_cast<size_t>(L) * M, 0);
  if (pool != nullptr) {
    hipError_t err = hipGetDevice(&c->device);
    const size_t n = static_cast<size_t>(L) * M;
    c->ready.assign(n, nullptr);
    c->released.assign(n, nullptr);
    c->ready_on.assign(n, 0);
    c->released_on.assign(n, 0);
    for (size_t i = 0; i < n && err == hipSuccess; ++i) {
      err = hipEventCreateWithFlags(&c->ready[i], hipEventDisableTiming);
      if (err == hipSuccess) err = hipEventCreateWithFlags(&c->released[i], hipEventDisableTiming);
    }
    if (err != hipSuccess) {
      smoe_status st = hip_fail(who, "event creation", err);
      for (hipEvent_t ev : c->ready)
        if (ev) (void)hipEventDestroy(ev);
      for (hipEvent_t ev : c->released)
        if (ev) (void)hipEventDestroy(ev);
      delete c;
      return st;
    }
  }
  *cache = c;
  return SMOE_OK;
}

extern "C" smoe_status smoe_cache_destroy(smoe_expert_cache* cache) {
  clear_error();
  if (cache == nullptr) return SMOE_OK;
  for (hipEvent_t ev : cache->ready)
    if (ev) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : cache->released)
    if (ev) (void)hipEventDestroy(ev);
  delete cache;
  return SMOE_OK;
}

extern "C" smoe_status smoe_cache_begin_window(smoe_expert_cache* cache) {
  clear_error();
  smoe_status st = check_cache(cache, "cache_begin_window");
  if (st != SMOE_OK) return st;
  std::fill(cache->claim.begin(), cache->claim.end(), 0);
  return SMOE_OK;
}

extern "C" smoe_status smoe_cache_state(const smoe_expert_cache* cache, int32_t* slot_expert,
                                        int64_t* last_use, int32_t* claimed, int64_t* clock) {
  clear_error();
  smoe_status st = check_cache(cache, "cache_state");
  if (st != SMOE_OK) return st;
  const size_t n = cache->held.size();
  for (size_t i = 0; i < n; ++i) {
    if (slot_expert) slot_expert[i] = cache->held[i];
    if (last_use) last_use[i] = cache->used[i];
    if (claimed) claimed[i] = cache->claim[i];
  }
  if (clock) *clock = cache->clock;
  return SMOE_OK;
}

extern "C" smoe_status smoe_cache_set_state(smoe_expert_cache* cache, const int32_t* slot_expert,
                                            const int64_t* last_use, int64_t clock,
                                            void* copy_stream) {
  clear_error();
  const char* who = "cache_set_state";
  smoe_status st = check_cache(cache, who);
  if (st != SMOE_OK) return st;
  SMOE_REQUIRE(slot_expert != nullptr && last_use != nullptr && clock >= 0, SMOE_EINVAL,
               "%s: null state or negative clock", who);
  const int L = cache->L, E = cache->E, M = cache->M;
  for (int l = 0; l < L; ++l) {
    std::vector<uint8_t> seen(E, 0);
    for (int s = 0; s < M; ++s) {
      const int e = slot_expert[l * M + s];
      SMOE_REQUIRE(e >= -1 && e < E, SMOE_EINVAL, "%s: layer %d slot %d holds expert %d", who,
                   l, s, e);
      SMOE_REQUIRE(e < 0 || !seen[e], SMOE_EINVAL, "%s: layer %d holds expert %d twice", who, l,
                   e);
      if (e >= 0) seen[e] = 1;
      SMOE_REQUIRE(last_use[l * M + s] >= 0 && last_use[l * M + s] <= clock, SMOE_EINVAL,
                   "%s: last use outside [0, clock]", who);
    }
  }
  std::fill(cache->where.begin(), cache->where.end(), -1);
  for (int l = 0; l < L; ++l)
    for (int s = 0; s < M; ++s) {
      cache->held[l * M + s] = -1;
      place(cache, l, s, slot_expert[l * M + s]);
      cache->used[l * M + s] = last_use[l * M + s];
    }
  std::fill(cache->claim.begin(), cache->claim.end(), 0);
  cache->clock = clock;
  if (device_mode(cache)) {
    hipStream_t io = as_stream(copy_stream);
    for (int l = 0; l < L; ++l)
      for (int s = 0; s < M; ++s) {
        const int e = cache->held[l * M + s];
        if (e < 0) continue;
        st = enqueue_load(cache, l, e, s, io, who);
        if (st != SMOE_OK) return st;
      }
  }
  return SMOE_OK;
}

extern "C" smoe_status smoe_cache_prefetch(smoe_expert_cache* cache, const int32_t* plan_ids,
                                           const int32_t* plan_counts, int plan_M,
                                           int32_t* loads, int* n_loads, int* full,
                                           void* copy_stream) {
  clear_error();
  const char* who = "cache_prefetch";
  smoe_status st = check_cache(cache, who);
  if (st != SMOE_OK) return st;
  SMOE_REQUIRE(plan_M >= 0 && (plan_M == 0 || (plan_ids && plan_counts)) && loads && n_loads,
               SMOE_EINVAL, "%s: null argument or negative plan_M", who);
  const int L = cache->L, E = cache->E, M = cache->M;
  for (int i = 0; i < L * plan_M; ++i)
    SMOE_REQUIRE(plan_ids[i] >= 0 && plan_ids[i] < E, SMOE_EINVAL,
                 "%s: plan entry %d names expert %d of %d", who, i, plan_ids[i], E);
  int n = 0;
  std::vector<int> order;
  std::vector<uint8_t> skip(M);
  for (int l = 0; l < L; ++l) {
    // the layer's selection: ranked experts with a positive count, at most M
    std::vector<int> sel;
    for (int m = 0; m < plan_M && static_cast<int>(sel.size()) < M; ++m)
      if (plan_counts[l * plan_M + m] > 0) sel.push_back(plan_ids[l * plan_M + m]);
    const int64_t now = ++cache->clock;
    for (int e : sel) {  // cached experts first: they keep their slots
      const int s = cache->where[l * E + e];
      if (s < 0) continue;
      cache->claim[l * M + s] = 1;
      cache->used[l * M + s] = now;
    }
    for (int e : sel) {
      if (cache->where[l * E + e] >= 0) continue;
      for (int s = 0; s < M; ++s) skip[s] = cache->claim[l * M + s];
      victim_order(cache, l, skip, order);
      if (order.empty()) break;  // every slot of the layer is claimed
      const int s = order[0];
      loads[4 * n + 0] = l;
      loads[4 * n + 1] = e;
      loads[4 * n + 2] = s;
      loads[4 * n + 3] = cache->held[l * M + s];
      ++n;
      place(cache, l, s, e);
      cache->claim[l * M + s] = 1;
      cache->used[l * M + s] = now;
      if (device_mode(cache)) {
        st = enqueue_load(cache, l, e, s, as_stream(copy_stream), who);
        if (st != SMOE_OK) return st;
      }
    }
  }
  *n_loads = n;
  if (full) {
    int f = 1;
    for (size_t i = 0; i < cache->claim.size() && f; ++i) f = cache->claim[i] != 0;
    *full = f;
  }
  return SMOE_OK;
}

extern "C" smoe_status smoe_prefetch_next_boundary(int b, int K, int n_transfer,
                                                   double expert_bytes, double h2d_gb_per_s,
                                                   double draft_us_per_token, int* next_b) {
  clear_error();
  const char* who = "prefetch_next_boundary";
  SMOE_REQUIRE(next_b != nullptr && b >= 0 && K >= b && n_transfer >= 0 && expert_bytes >= 0 &&
                   h2d_gb_per_s > 0 && draft_us_per_token > 0,
               SMOE_EINVAL,
               "%s: need 0 <= b <= K, n_transfer >= 0, expert_bytes >= 0 and positive "
               "bandwidth and draft time", who);
  // transfer time in microseconds, then the chunk whose draft time covers it
  const double t_io = n_transfer * expert_bytes / (h2d_gb_per_s * 1000.0);
  const double chunks = std::ceil(t_io / draft_us_per_token);
  const long long n = std::max(1ll, static_cast<long long>(std::min(chunks, 1e9)));
  *next_b = static_cast<int>(std::min<long long>(b + n, K));
  return SMOE_OK;
}

extern "C" smoe_status smoe_cache_verify_plan(smoe_expert_cache* cache, int layer,
                                              const int32_t* expert_counts, int32_t* schedule,
                                              int* n_schedule) {
  clear_error();
  const char* who = "cache_verify_plan";
  smoe_status st = check_cache(cache, who);
  if (st != SMOE_OK) return st;
  SMOE_REQUIRE(layer >= 0 && layer < cache->L && expert_counts && schedule && n_schedule,
               SMOE_EINVAL, "%s: bad layer %d or null argument", who, layer);
  std::vector<Step> steps;
  st = verify_decide(cache, layer, expert_counts, steps, who);
  if (st != SMOE_OK) return st;
  for (size_t i = 0; i < steps.size(); ++i) {
    schedule[5 * i + 0] = steps[i].expert;
    schedule[5 * i + 1] = steps[i].slot;
    schedule[5 * i + 2] = steps[i].kind;
    schedule[5 * i + 3] = steps[i].evicted;
    schedule[5 * i + 4] = steps[i].wait;
  }
  *n_schedule = static_cast<int>(steps.size());
  return SMOE_OK;
}

extern "C" smoe_status smoe_cache_verify_layer(
    smoe_expert_cache* cache, int layer, const int32_t* expert_counts, const void* x, int T,
    int k, int H, int I, int tiled, const int32_t* sorted_slots, const int32_t* expert_offsets,
    int shared_I, const void* shared_wg, const void* shared_wu, const void* shared_wd,
    void* workspace_shared, size_t workspace_shared_bytes, void* workspace_routed,
    size_t workspace_routed_bytes, float* slot_out, float* shared_out, int32_t* schedule,
    int* n_schedule, void* compute_stream, void* copy_stream) {
  clear_error();
  const char* who = "cache_verify_layer";
  smoe_status st = check_cache(cache, who);
  if (st != SMOE_OK) return st;
  SMOE_REQUIRE(device_mode(cache), SMOE_EINVAL,
               "%s: the cache was created without device memory", who);
  SMOE_REQUIRE(layer >= 0 && layer < cache->L && expert_counts != nullptr, SMOE_EINVAL,
               "%s: bad layer %d or null expert_counts", who, layer);
  SMOE_REQUIRE(H > 0 && I > 0 &&
                   cache->expert_bytes == 3ull * static_cast<size_t>(H) * I * sizeof(uint16_t),
               SMOE_EINVAL, "%s: expert_bytes %zu is not that of three fp16 %d x %d matrices",
               who, cache->expert_bytes, I, H);
  SMOE_REQUIRE(workspace_routed != nullptr && (shared_I == 0 || workspace_shared != nullptr),
               SMOE_EINVAL, "%s: null workspace", who);
  SMOE_REQUIRE(shared_I == 0 || workspace_shared != workspace_routed, SMOE_EINVAL,
               "%s: with shared experts the two workspaces must differ (they serve different "
               "shapes)", who);
  const int L = cache->L, E = cache->E, M = cache->M;
  const long long n_mat_ll = 3ll * L * M - 2;
  SMOE_REQUIRE(n_mat_ll > 0 && n_mat_ll < (1ll << 31), SMOE_EUNSUPPORTED,
               "%s: the pool holds too many matrices", who);
  const int n_mat = static_cast<int>(n_mat_ll);
  const size_t msz = static_cast<size_t>(I) * H * sizeof(uint16_t);
  const uint8_t* wg = cache->pool;
  const uint8_t* wu = cache->pool + msz;
  const uint8_t* wd = cache->pool + 2 * msz;
  // the decisions, on a copy of the state: nothing changes if a check fails
  std::vector<Step> steps;
  {
    Cache trial = *cache;
    trial.ready.clear();
    trial.released.clear();
    st = verify_decide(&trial, layer, expert_counts, steps, who);
    if (st != SMOE_OK) return st;
  }
  // the launches' own checks, before anything is enqueued
  SMOE_REQUIRE(T >= 0 && k > 0 && k <= kMaxK && shared_I >= 0 && H % 128 == 0 && I % 128 == 0 &&
                   shared_I % 128 == 0 && (tiled == 0 || tiled == 1),
               SMOE_EINVAL,
               "%s: need T >= 0, 0 < k <= 8, H, I and shared_I multiples of 128, tiled 0 or 1 "
               "(T=%d k=%d H=%d I=%d shared_I=%d tiled=%d)", who, T, k, H, I, shared_I, tiled);
  SMOE_REQUIRE(T == 0 || (x && sorted_slots && expert_offsets && slot_out &&
                          (shared_I == 0 || (shared_wg && shared_wu && shared_wd && shared_out))),
               SMOE_EINVAL, "%s: null pointer", who);
  SMOE_REQUIRE(workspace_routed_bytes >= smoe_ffn_workspace_bytes(T, k, E, H, I, 0) &&
                   (shared_I == 0 ||
                    workspace_shared_bytes >= smoe_ffn_workspace_bytes(T, k, E, H, I, shared_I)),
               SMOE_EINVAL, "%s: a workspace is smaller than smoe_ffn_workspace_bytes", who);
  std::vector<int32_t> table(E, -1);
  steps.clear();
  st = verify_decide(cache, layer, expert_counts, steps, who);
  if (st != SMOE_OK) return st;
  hipStream_t cs = as_stream(compute_stream), io = as_stream(copy_stream);
  auto slot_index = [&](int s) { return static_cast<size_t>(layer) * M + s; };
  auto after_compute = [&](int s) -> smoe_status {
    hipError_t err = hipEventRecord(cache->released[slot_index(s)], cs);
    if (err != hipSuccess) return hip_fail(who, "hipEventRecord", err);
    cache->released_on[slot_index(s)] = 1;
    return SMOE_OK;
  };
  auto before_compute = [&](int s) -> smoe_status {
    if (!cache->ready_on[slot_index(s)]) return SMOE_OK;
    hipError_t err = hipStreamWaitEvent(cs, cache->ready[slot_index(s)], 0);
    return err == hipSuccess ? SMOE_OK : hip_fail(who, "hipStreamWaitEvent", err);
  };
  auto mat_of = [&](int s) { return static_cast<int32_t>(3 * slot_index(s)); };
  // the hits (and the always-on shared experts) in one computation
  size_t i = 0;
  bool any_hit = false;
  for (; i < steps.size() && steps[i].kind == kHit; ++i) {
    table[steps[i].expert] = mat_of(steps[i].slot);
    any_hit = true;
    if ((st = before_compute(steps[i].slot)) != SMOE_OK) return st;
  }
  if (any_hit || shared_I > 0) {
    st = smoe_fp16_expert_ffn_mapped(x, T, k, E, H, I, wg, wu, wd, tiled, n_mat, table.data(),
                                     sorted_slots, expert_offsets, shared_I, shared_wg,
                                     shared_wu, shared_wd,
                                     shared_I ? workspace_shared : workspace_routed,
                                     shared_I ? workspace_shared_bytes : workspace_routed_bytes,
                                     slot_out, shared_out, compute_stream);
    if (st != SMOE_OK) return st;
    for (size_t h = 0; h < i; ++h)
      if ((st = after_compute(steps[h].slot)) != SMOE_OK) return st;
  }
  // each miss: its copy after the slot's last reader, its computation after
  // the copy
  for (; i < steps.size(); ++i) {
    const Step& m = steps[i];
    if ((st = enqueue_load(cache, layer, m.expert, m.slot, io, who)) != SMOE_OK) return st;
    if ((st = before_compute(m.slot)) != SMOE_OK) return st;
    std::fill(table.begin(), table.end(), -1);
    table[m.expert] = mat_of(m.slot);
    st = smoe_fp16_expert_ffn_mapped(x, T, k, E, H, I, wg, wu, wd, tiled, n_mat, table.data(),
                                     sorted_slots, expert_offsets, 0, nullptr, nullptr, nullptr,
                                     workspace_routed, workspace_routed_bytes, slot_out, nullptr,
                                     compute_stream);
    if (st != SMOE_OK) return st;
    if ((st = after_compute(m.slot)) != SMOE_OK) return st;
  }
  if (schedule != nullptr) {
    for (size_t j = 0; j < steps.size(); ++j) {
      schedule[5 * j + 0] = steps[j].expert;
      schedule[5 * j + 1] = steps[j].slot;
      schedule[5 * j + 2] = steps[j].kind;
      schedule[5 * j + 3] = steps[j].evicted;
      schedule[5 * j + 4] = steps[j].wait;
    }
  }
  if (n_schedule != nullptr) *n_schedule = static_cast<int>(steps.size());
  return SMOE_OK;
}
