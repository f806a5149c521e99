// Long-window expert FFN over tiled weights: the fused multi-expert FFN when
// a window holds many tokens per expert (batched speculative windows: tens
// of slots per expert), so that each expert's weights should stream once
// per chunk of its slots rather than once per few slots.
//
// Specter paper: expert-wise verification paragraphs (the tokens of an
// expert form one dense sub-batch, turning GEMVs into GEMMs; outputs go back
// to their slots), fused multi-expert draft kernel paragraph (every active
// expert in one launch) and the batched-execution paragraph (up to 32
// requests per step); hybrid-precision layout (FP16 shared experts). Design
// notes, "Streamlined Execution Engine": INT4 tiles dequantised inside the
// GEMM with FP16 activations and FP32 reductions.
//
// Two launches over all active routed experts and the optional FP16 shared
// expert:
//   stage 1  h[p] = fp16( SiLU(x_t . Wg^T) * (x_t . Wu^T) )   (p = sorted position)
//   stage 2  out[s] = h[p] . Wd^T                             (s = sorted_slots[p])
// An item is (chunk of up to 16*NC positions of one expert, tile of 128
// output rows) and is computed over the whole reduction length by one
// workgroup: eight waves each own 16 rows of the tile (in stage 1 the same
// 16 rows of gate and of up, so SiLU(g) * u is formed in registers and h is
// written once, in fp16), so no sum is split between waves or workgroups:
// no atomics, nothing to clear, the same result on every run.
//
// Four more waves stage the item's activation rows into LDS, k-phase by
// k-phase (double-buffered; the hand-over is a pair of step counters in LDS,
// not a barrier), while the eight stream their weight rows through a
// register ring of R blocks that runs on across phases and items (the
// streamers never wait on anything but their oldest weight block and the
// step counter of the buffer they read). INT4 and FP16 weights come tiled
// (smoe_tile_weights): one wave load reads 16 rows x 64 bytes in one piece.
//
// Work split, computed on the device from the expert offsets (nothing read
// back): the shared expert's items are cut into contiguous ranges over the
// first workgroups, balanced by the weight blocks a wave streams per item;
// the routed items (chunk by chunk, tile by tile) are claimed one at a time
// at run time from a counter in the workspace, so that a workgroup that
// drew cheap items takes more. When a launch has more than 16 items per
// workgroup (past what the LDS item tables are sized for), every item is
// cut into static ranges instead.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "ffn_device.hpp"
#include "ffn_wide.hpp"

namespace smoe {
namespace {

constexpr int kWW = 8;                        // streamer waves
constexpr int kWS = 4;                        // staging waves
constexpr int kWThreads = (kWW + kWS) * kWave;
constexpr int kWLds = 160 * 1024;             // one workgroup per CU (gfx950)
constexpr int kWPad = 16;                     // bytes of padding per staged row
constexpr int kWStageNB = 16;                 // staging loads in flight per lane
#ifndef SMOE_WIDE_RING
#define SMOE_WIDE_RING 4
#endif
constexpr int kWRing = SMOE_WIDE_RING;        // weight blocks in flight per streamer
constexpr int kWItems = 64;                   // items of a range in the LDS table
constexpr int kWTabInts = 2 * (kMaxE + 4) + kWideMaxSlots + 4 + 4 * kWItems;  // + step counters, items
constexpr int kWTabBytes = (kWTabInts * 4 + 15) / 16 * 16;
// Positions per chunk: 64 for the routed experts (4 MFMA column groups,
// k-phases of 512). The FP16 shared gate/up take 128 tokens (8 column
// groups, k-phases of 256), so that those weights stream half as often; the
// shared down rows take 64, as the routed ones: a 128-token item of the
// long shared K is several routed items long, and the workgroups that take
// them would finish well after the others. The INT4 kernels with 8 column
// groups would exceed the register budget of 12 waves per CU and spill.
constexpr int kNC0 = 4, kNC1 = 8;
constexpr int kKph0 = 512, kKph1 = 256;
// Routed down rows: each streamer wave takes two 16-row slabs of a 256-row
// tile, so a staged chunk of h rows serves twice the rows (the activations
// staged per weight byte halve).
constexpr int kSL0 = 2;

struct WGroup {
  const uint8_t* w[2];      // stage 1: gate, up; stage 2: down (w[1] = w[0])
  const uint16_t* s[2];     // INT4 scales (tiled), null for FP16
  long long w_estride;      // bytes per expert matrix
  long long s_estride;      // scale elements per expert matrix
  long long cost;           // work-split cost of one item
  int nblk;                 // 64-byte blocks per weight row
  int bpp;                  // blocks per staged k-phase
  int slabs;                // output rows / 16
  int tiles;                // ceil(slabs / (8 * slabs per wave))
  int K;                    // reduction length (elements)
  int ch;                   // positions per chunk
  int kph;                  // k per staged phase (elements)
  int rstride;              // LDS bytes per staged row
  const uint16_t* a;        // stage 1: x [T][H]; stage 2: this group's h [rows][K]
  void* out;                // stage 1: fp16 h [rows][N]; stage 2: fp32 [*][H]
};

struct WArgs {
  const int32_t* sorted_slots;
  const int32_t* offsets;
  float* slot_out;          // stage 2: rows of dropped slots are zeroed
  int E, k, S, T, H;
  int shared;               // group 1 (the FP16 shared expert) present
  int buf_bytes;            // LDS bytes per phase buffer
  int zero_dropped;         // stage 2: zero the slot_out rows of dropped slots
  int* claim;               // routed items claimed so far (zero at the launch), or null
  int* finished;            // workgroups done claiming (zero at the launch)
  WGroup g[2];              // 0: routed experts, 1: shared expert
};

typedef const __attribute__((address_space(4))) WArgs ConstWArgs;
__device__ __forceinline__ ConstWArgs* wkargs() {
  return (ConstWArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
}

// Workgroup barrier that orders LDS only: every barrier here hands over LDS
// data (tables); a full fence would wait for the weight loads in flight too.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The staged steps are handed over with counters in LDS instead of
// barriers: a staging wave adds one to ready[b] when its rows of a step are
// in buffer b, a streamer adds one to done[b] when it has read its last
// block of a step from buffer b. Each side waits only for what it needs,
// so the twelve waves do not meet at every step. A wait gives up after
// about 0.1 s (it cannot be reached unless a wave of the workgroup died).
constexpr int kStepSpin = 1 << 22;
__device__ __forceinline__ void step_wait(int* ctr, int target) {
  for (int i = 0; i < kStepSpin &&
                  __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target;
       ++i)
    __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ void step_signal(int* ctr, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");  // this wave's LDS accesses done
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<P*>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<I + 1, N>(f);
  }
}

// An item: (group, expert, first position, positions, tile); wave-uniform.
struct It {
  int grp, e, seg0, m, tile;
};

// What the streamer passes and the staging loop share.
struct WCtx {
  uint8_t* bufs;            // the two phase buffers
  const int* s_off;         // expert offsets, clamped to [0, S]
  const int* s_cp;          // routed chunks before each expert
  const int* s_slots;       // stage 1: token of each position; stage 2: its slot
  int* ready;               // [2] staging waves' step counters per buffer
  int* done;                // [2] streamers' step counters per buffer
  i32x4* items;             // the workgroup's items by local index (kWItems)
  int lo, ns;               // its static items: global lo + i for local i < ns
  int dyn;                  // routed items past the static ones are claimed at run time
  int* claim;               // the launch's claim and finish counters (dyn)
  int* finished;
  int n0;                   // routed items
  int nwg;
  int ph0, ph1;             // staged steps per item of each group
  int n1;                   // shared items (they come first)
  int E, T;
  int wave, lane;
};

// The item's fields, decoded by one lane on its own (a binary search over
// the routed chunk prefix).
__device__ __forceinline__ It decode_item(const WCtx& c, int item) {
  ConstWArgs* ka = wkargs();
  It it;
  if (item < c.n1) {
    const int tiles1 = ka->g[1].tiles, ch1 = ka->g[1].ch;
    const int ck = item / tiles1;
    it.grp = 1;
    it.e = 0;
    it.tile = item - ck * tiles1;
    it.seg0 = ck * ch1;
    it.m = min(ch1, c.T - it.seg0);
  } else {
    const int tiles0 = ka->g[0].tiles, ch0 = ka->g[0].ch;
    const int ri = item - c.n1;
    const int rc = ri / tiles0;
    it.grp = 0;
    it.tile = ri - rc * tiles0;
    int e = 0, hi_e = c.E;  // s_cp[e] <= rc < s_cp[hi_e]
    while (hi_e - e > 1) {
      const int mid = (e + hi_e) >> 1;
      if (c.s_cp[mid] <= rc) e = mid; else hi_e = mid;
    }
    it.e = e;
    it.seg0 = c.s_off[e] + (rc - c.s_cp[e]) * ch0;
    it.m = min(ch0, c.s_off[e + 1] - it.seg0);
  }
  return it;
}

// Table entries of items not claimed yet, and the entry after the last item.
constexpr int kPending = -2, kEnd = -1;
constexpr int kClaimSpin = 1 << 22;

// Whether the workgroup's local item i exists: a static item, or a claimed
// one (waits until the claiming wave has written the entry; a wait that
// gives up, which only a dead wave could cause, reads as the end).
__device__ __forceinline__ bool item_valid(const WCtx& c, int i) {
  if (i < c.ns) return true;
  if (!c.dyn || i >= kWItems) return false;
  int v = kPending;
  for (int n = 0; n < kClaimSpin; ++n) {
    v = __hip_atomic_load(reinterpret_cast<int*>(c.items + i), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_WORKGROUP);
    if (v != kPending) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return uniform(v) >= 0;
}

// The fields of the workgroup's local item i (valid) for the whole wave:
// from the table, or (static items past its end) decoded here.
__device__ __forceinline__ It item_at(const WCtx& c, int i) {
  It it;
  if (i < kWItems) {
    const i32x4 v = c.items[i];
    it.grp = v[0] >> 16;
    it.e = v[0] & 0xFFFF;
    it.seg0 = v[1];
    it.m = v[2];
    it.tile = v[3];
  } else {
    it = decode_item(c, c.lo + i);
  }
  it.grp = uniform(it.grp);
  it.e = uniform(it.e);
  it.seg0 = uniform(it.seg0);
  it.m = uniform(it.m);
  it.tile = uniform(it.tile);
  return it;
}


// The staging waves: every (item, phase) of the workgroup's items in order,
// into the buffer of its step's parity. With run-time claims, the first
// staging wave also claims the routed items and writes them into the item
// table. Lane c of a
// staging wave copies the 16-byte piece c of every fourth row (a row of a
// phase is at most 64 pieces), so a piece costs an add for its address and
// a row's token is looked up once.
template <int STAGE>
__device__ __forceinline__ void staging_loop(const WCtx& c) {
  ConstWArgs* ka = wkargs();
  const int ws = c.wave - kWW;
  const int lane = c.lane;
  // the launch's values, read once into scalar registers
  const int buf_bytes = uniform(ka->buf_bytes);
  const int K0 = uniform(ka->g[0].K), K1 = uniform(ka->g[1].K);
  const int kph0 = uniform(ka->g[0].kph), kph1 = uniform(ka->g[1].kph);
  const int rs0 = uniform(ka->g[0].rstride), rs1 = uniform(ka->g[1].rstride);
  const uint16_t* const a0 = uniform_ptr(ka->g[0].a);
  const uint16_t* const a1 = uniform_ptr(ka->g[1].a);
  const int S = uniform(ka->S);
  // A step is staged in two parts. The first batch of rows (kWStageNB rows
  // per wave, all of a 64-row chunk) is loaded into registers before the
  // wave waits for its buffer to be free, so the loads' round trip overlaps
  // the streamers' use of that buffer; the rest (rows past the batch) is
  // loaded and written after.
  struct Src {
    const uint16_t* src;  // this lane's piece in row 0 of the source
    int K, rstride, rows;
    bool on;              // the lane holds a piece of this phase
  };
  auto src_of = [&](const It& it, int p) __attribute__((always_inline)) {
    Src q;
    q.K = it.grp ? K1 : K0;
    const int kph = it.grp ? kph1 : kph0;
    q.rstride = it.grp ? rs1 : rs0;
    const int k0 = p * kph;
    const int npr = min(kph, q.K - k0) / 8;  // 16-byte pieces per row
    q.src = (it.grp ? a1 : a0) + k0 + 8 * min(lane, npr - 1);
    q.on = lane < npr;
    q.rows = STAGE == 1 ? c.T : (it.grp ? c.T : S);  // rows of the source
    return q;
  };
  auto load_rows = [&](const It& it, const Src& q, int r0, u32x4 (&v)[kWStageNB])
      __attribute__((always_inline)) {
    static_for<0, kWStageNB>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int r = min(r0 + j * kWS, it.m - 1);
      int row = (STAGE == 1 && !it.grp) ? uniform(c.s_slots[it.seg0 + r]) : it.seg0 + r;
      row = min(max(row, 0), q.rows - 1);
      v[j] = gload<u32x4>(q.src + static_cast<long long>(row) * q.K);
    });
  };
  auto store_rows = [&](const It& it, const Src& q, int r0, int buf, const u32x4 (&v)[kWStageNB])
      __attribute__((always_inline)) {
    uint8_t* dst0 = c.bufs + buf * buf_bytes + 16 * lane;
    static_for<0, kWStageNB>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int r = r0 + j * kWS;
      if (q.on && r < it.m) *reinterpret_cast<u32x4*>(dst0 + r * q.rstride) = v[j];
    });
  };
  auto stage_rest = [&](const It& it, const Src& q, int buf) __attribute__((always_inline)) {
    for (int r0 = ws + kWS * kWStageNB; r0 < it.m; r0 += kWS * kWStageNB) {
      u32x4 v[kWStageNB];
      load_rows(it, q, r0, v);
      store_rows(it, q, r0, buf, v);
    }
  };
  // claims of local items up to i (first staging wave): one device-scope
  // add per item; the claim that finds no item left ends the workgroup's
  // claims, and the last workgroup to end them sets the two counters back
  // to zero for the next launch
  int claimed = c.ns;
  bool over = false;
  auto claim_upto = [&](int i) __attribute__((always_inline)) {
    if (!c.dyn || ws != 0 || over) return;
    while (claimed <= i) {
      int k = c.n0;  // (the table is full: no claim)
      if (claimed < kWItems - 1) {
        int kk = 0;
        if (lane == 0)
          kk = __hip_atomic_fetch_add(c.claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        k = uniform(kk);
      }
      int* entry = reinterpret_cast<int*>(c.items + claimed);
      if (k < c.n0) {
        if (lane == 0) {
          const It nt = decode_item(c, c.n1 + k);
          entry[1] = nt.seg0;
          entry[2] = nt.m;
          entry[3] = nt.tile;
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
          __hip_atomic_store(entry, nt.e | (nt.grp << 16), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        ++claimed;
      } else {
        int f = 0;
        if (lane == 0) {
          __hip_atomic_store(entry, kEnd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          f = __hip_atomic_fetch_add(c.finished, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (f == c.nwg - 1) {
            __hip_atomic_store(c.claim, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(c.finished, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        over = true;
        break;
      }
    }
  };
  // An item is claimed right after the previous one's last phase is staged
  // (so the claim's round trip does not delay that phase): the streamers'
  // loads, R <= 2 blocks ahead of their MFMAs, reach it only after that
  // phase's step has begun, and a workgroup holds little claimed work it
  // has not started when the counter runs out.
  claim_upto(0);
  if (!item_valid(c, 0)) return;
  int step = 0;
  It it = item_at(c, 0);
  int p = 0;
  u32x4 v[kWStageNB];
  {
    const Src q = src_of(it, 0);
    load_rows(it, q, ws, v);
    store_rows(it, q, ws, 0, v);
    stage_rest(it, q, 0);
  }
  step_signal(c.ready, lane);
  if ((it.grp ? c.ph1 : c.ph0) == 1) claim_upto(1);
  for (int item = 0;;) {
    // the next step: next phase of this item, or the next item's first
    int nitem = item, np = p + 1;
    if (np >= (it.grp ? c.ph1 : c.ph0)) {
      ++nitem;
      np = 0;
      if (!item_valid(c, nitem)) break;
    }
    const It nit = nitem == item ? it : item_at(c, nitem);
    const int s1 = step + 1, b = s1 & 1;
    const Src q = src_of(nit, np);
    load_rows(nit, q, ws, v);  // in flight while the buffer is still read
    if (s1 >= 2) step_wait(c.done + b, kWW * (s1 >> 1));  // steps s1 - 2, s1 - 4, ... read
    store_rows(nit, q, ws, b, v);
    stage_rest(nit, q, b);
    step_signal(c.ready + b, lane);
    if (np == (nit.grp ? c.ph1 : c.ph0) - 1) claim_upto(nitem + 1);
    item = nitem;
    p = np;
    it = nit;
    ++step;
  }
}

// One streamer wave over the local items [first, last) (last < 0: up to the
// first local item that does not exist, claimed at run time), all of group
// GRP, whose
// weights are in format FMT: NC column groups of 16 positions against 16
// rows of each weight stream over the whole reduction length. In stage 1
// the streams are the gate and up rows of slab tile * 8 + wave; in stage 2
// they are the down rows of SL slabs, (tile * SL + j) * 8 + wave, so that
// one staged chunk serves SL times the rows. `step` counts the staged steps
// of the workgroup (the parity picks the buffer); it runs on from one pass
// to the next.
template <int FMT, int G, int STAGE, int NC, int GRP, int SL>
__device__ __forceinline__ void stream_pass(const WCtx& c, int first, int last, int& step) {
  constexpr int NMAT = STAGE == 1 ? 2 : SL;  // weight streams
  constexpr int NQ = FMT == kInt4 ? 128 / G : 1;  // INT4 scales per block and row
  constexpr int NS = NQ == 4 ? 2 : 1;
  constexpr int PER = G / 32;                     // MFMA steps per INT4 group
  ConstWArgs* ka = wkargs();
  const int wave = c.wave;
  // the lane's own copy in this pass: values derived from it are formed
  // here, not kept live from the workgroup's other pass
  int lane = c.lane;
  asm volatile("" : "+v"(lane));
  const int g = lane >> 4;
  const int r16 = lane & 15;
  // the launch's values, read once into scalar registers (the compiler
  // would otherwise load them from the argument segment again inside the
  // loop, each load a wait on the scalar and LDS counters)
  const int nblk = uniform(ka->g[GRP].nblk), bpp = uniform(ka->g[GRP].bpp);
  const int slabs = uniform(ka->g[GRP].slabs);
  const int rstride = uniform(ka->g[GRP].rstride);
  const int buf_bytes = uniform(ka->buf_bytes);
  const int H = uniform(ka->H), S = uniform(ka->S);
  const long long west = ka->g[GRP].w_estride;
  const long long sest = ka->g[GRP].s_estride;
  const uint8_t* const wbase[2] = {uniform_ptr(ka->g[GRP].w[0]), uniform_ptr(ka->g[GRP].w[1])};
  const uint16_t* const sbase[2] = {uniform_ptr(ka->g[GRP].s[0]), uniform_ptr(ka->g[GRP].s[1])};
  void* const out = uniform_ptr(ka->g[GRP].out);

  auto slab_of = [&](int tile, int m) __attribute__((always_inline)) {
    return STAGE == 1 ? tile * kWW + wave : (tile * SL + m) * kWW + wave;
  };
  struct Cur {  // the load cursor: a position in the wave's block sequence (wave-uniform)
    int item, blk;
    bool done;                // past the last item
    const uint8_t* w[NMAT];   // each stream's current block
    const uint16_t* s[NMAT];  // and its scales (INT4)
  };
  auto settle = [&](Cur& cu) __attribute__((always_inline)) {  // at the start of item cu.item (< hi)
    const It it = item_at(c, cu.item);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      // (slabs past N: loaded, never stored)
      const long long tb0 = static_cast<long long>(min(slab_of(it.tile, m), slabs - 1)) * nblk;
      const int mat = STAGE == 1 ? m : 0;
      cu.w[m] = wbase[mat] + it.e * west + tb0 * 1024;
      if (FMT == kInt4) cu.s[m] = sbase[mat] + it.e * sest + tb0 * 16 * NQ;
    }
    cu.blk = 0;
  };

  struct Entry {
    u32x4 v[NMAT];
    uint32_t s[NMAT][NS];
    uint16_t s16[NMAT];
  };
  constexpr int R = kWRing / NMAT;  // ring entries: kWRing weight blocks in flight
  // The load cursor runs R blocks ahead; a routed item is claimed once the
  // previous item's last phase is staged, which covers it when R <= 2.
  static_assert(GRP == 1 || R <= 2, "a claimed item must be in the table before the loads reach it");
  Entry ring[R];
  // Every ring slot takes a load on every pass, also past the end of the
  // range (the last block again), so that the compiler waits only for the
  // oldest block.
  const uint32_t lane16 = 16 * lane;   // this lane's bytes of a block
  const uint32_t srow = r16 * NQ;      // and its row's scales
  auto load = [&](Entry& en, const Cur& cu) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      en.v[m] = gload<u32x4>(cu.w[m] + lane16);
      if (FMT == kInt4) {
        const uint16_t* sp = cu.s[m] + srow;
        if (NQ == 1) {
          en.s16[m] = gload<uint16_t>(sp);
        } else if (NQ == 2) {
          en.s[m][0] = gload<uint32_t>(sp);
        } else {
          const u32x2 v2 = gload<u32x2>(sp);
          en.s[m][0] = v2[0];
          en.s[m][NS - 1] = v2[1];
        }
      }
    }
  };
  // the next block; past the end of the range the cursor stays on the last
  // block (it is loaded again, never computed)
  int c_end = last >= 0 ? last : 0x7FFFFFFF;  // the first local item past the range
  auto advance = [&](Cur& cu) __attribute__((always_inline)) {
    if (cu.blk + 1 < nblk) {
      ++cu.blk;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        cu.w[m] += 1024;
        if (FMT == kInt4) cu.s[m] += 16 * NQ;
      }
    } else if (!cu.done) {
      if (last >= 0 ? cu.item + 1 < last : item_valid(c, cu.item + 1)) {
        ++cu.item;
        settle(cu);
      } else {
        cu.done = true;
        c_end = cu.item + 1;  // before the compute cursor gets there (it is R blocks behind)
      }
    }
  };

  f32x4 acc[NMAT][NC];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) acc[m][cg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t dq_lo = 0x000F000Fu, dq_hi = 0x00F000F0u, dq_magic = 0x64006400u;
  asm volatile("" : "+v"(dq_lo), "+v"(dq_hi), "+v"(dq_magic));  // keep the masks in VGPRs

  int arow[NC];  // A-operand rows of this lane in the current buffer (LDS bytes)
  int cur_m = 0;
  It cit;        // the item being computed
  auto set_rows = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
      const int r = min(16 * cg + r16, max(cur_m - 1, 0));
      arow[cg] = buf * buf_bytes + r * rstride;
    }
  };
  auto lds16 = [&](int off) __attribute__((always_inline)) -> f16x8 {
    return *reinterpret_cast<const f16x8*>(c.bufs + off);
  };
  // one block at k offset kk within the phase. Every column group is
  // computed, also past the chunk's positions (their rows repeat the last
  // staged one and are never stored): with a run-time skip per column group
  // between the MFMAs, the g32 kernels gave wrong rows at a ring depth of
  // four blocks, and without the branches they do not.
  // The INT4 path sits behind a run-time test that always holds, and its
  // column groups behind scheduling barriers: without them the compiler
  // interleaves the dequantisation of consecutive blocks and the INT4
  // passes spill.
  const bool int4_rt = bpp > 0;
  auto compute = [&](const Entry& en, int kk) __attribute__((always_inline)) {
    // The activation fragments of column group cg + 1 are read from LDS
    // before the MFMAs of cg, so that the LDS latency hides behind them.
    if (FMT == kInt4 && int4_rt) {
      f16x8 B[NMAT][4];
      float sc[NMAT][NQ];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
#pragma unroll
        for (int q = 0; q < 4; ++q) B[m][q] = dequant_word(en.v[m][q], dq_lo, dq_hi, dq_magic);
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) {
          uint16_t sbits;
          if (NQ == 1) {
            sbits = en.s16[m];
          } else {
            const uint32_t word = en.s[m][NQ == 4 ? (gq >> 1) : 0];
            sbits = static_cast<uint16_t>((gq & 1) ? (word >> 16) : word);
          }
          sc[m][gq] = static_cast<float>(bitcast<_Float16>(sbits));
        }
      }
      f16x8 A[2][4];
      auto read_a = [&](int cg) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          A[cg & 1][q] = lds16(arow[cg] + 2 * (kk + 8 * int4_word(G, g, q)));
      };
      read_a(0);
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) {
        if (cg + 1 < NC) read_a(cg + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int qq = 0; qq < PER; ++qq) {
              const int q = gq * PER + qq;
              t = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[cg & 1][q], B[m][q], t, 0, 0, 0);
            }
            acc[m][cg] += sc[m][gq] * t;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      f16x8 A[2];
      A[0] = lds16(arow[0] + 2 * (kk + 8 * g));
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) {
        if (cg + 1 < NC) A[(cg + 1) & 1] = lds16(arow[cg + 1] + 2 * (kk + 8 * g));
        if (NC > 4) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
          acc[m][cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[cg & 1], bitcast<f16x8>(en.v[m]),
                                                              acc[m][cg], 0, 0, 0);
        if (NC > 4) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // outputs of the finished item cit, then the accumulators back to zero
  auto item_end = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < (STAGE == 1 ? 1 : NMAT); ++j) {
      const int slab = slab_of(cit.tile, j);
      if (slab >= slabs) continue;
      const int n = slab * 16 + r16;
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * cg + 4 * g + i;
          if (r >= cit.m) continue;
          if (STAGE == 1) {
            const int N = slabs * 16;
            const float gv = acc[0][cg][i], uv = acc[1][cg][i];
            const float h = gv / (1.0f + __expf(-gv)) * uv;
            gstore<_Float16>(static_cast<_Float16*>(out) +
                                 static_cast<long long>(cit.seg0 + r) * N + n,
                             static_cast<_Float16>(h));
          } else {
            const int row = GRP ? cit.seg0 + r : c.s_slots[cit.seg0 + r];
            if (row < 0 || row >= (GRP ? c.T : S)) continue;
            gstore<float>(static_cast<float*>(out) + static_cast<long long>(row) * H + n,
                          acc[j][cg][i]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) acc[m][cg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  };
  // before the first block of a step: the step's barrier and A rows
  // the compute cursor: item, block and block within the phase
  int c_item = first, c_blk = 0, c_bip = 0;
  auto begin_step = [&]() __attribute__((always_inline)) {
    if (c_blk == 0) {
      if (c_item != first) item_end();
      cit = item_at(c, c_item);
      cur_m = cit.m;
    }
    if (step > 0) step_signal(c.done + ((step - 1) & 1), lane);  // step - 1 read
    step_wait(c.ready + (step & 1), kWS * ((step >> 1) + 1));
    set_rows(step & 1);
    ++step;
  };

  auto advance_comp = [&]() __attribute__((always_inline)) {
    if (++c_blk == nblk) {
      c_blk = 0;
      c_bip = 0;
      ++c_item;
    } else if (++c_bip == bpp) {
      c_bip = 0;
    }
  };
  Cur L;
  L.item = first;
  L.done = false;
  settle(L);
  static_for<0, R>([&](auto rc) {
    load(ring[decltype(rc)::value], L);
    advance(L);
  });
  constexpr int kBlkK = FMT == kInt4 ? 128 : 32;  // k per block
  // While the load cursor is inside the range, the R blocks in the ring all
  // lie before it: R blocks a round, no checks. Then at most R are left.
  while (!L.done) {
    static_for<0, R>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      if (c_bip == 0) begin_step();
      compute(ring[r], c_bip * kBlkK);
      load(ring[r], L);
      advance(L);
      advance_comp();
    });
  }
  static_for<0, R>([&](auto rc) {
    constexpr int r = decltype(rc)::value;
    if (c_item < c_end) {
      if (c_bip == 0) begin_step();
      compute(ring[r], c_bip * kBlkK);
      advance_comp();
    }
  });
  item_end();
}

template <int WK, int G, int STAGE>
__global__ __launch_bounds__(kWThreads, 1) void wide_ffn_kernel(WArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  int* s_off = reinterpret_cast<int*>(smem);
  int* s_cp = s_off + kMaxE + 4;
  int* s_slots = s_off + 2 * (kMaxE + 4);
  int* s_steps = s_slots + kWideMaxSlots;  // ready[2], done[2]
  i32x4* s_items = reinterpret_cast<i32x4*>(s_steps + 4);
  uint8_t* bufs = smem + kWTabBytes;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int E = a.E;
  const int b = blockIdx.x;
  const int nwg = gridDim.x;

  // ---- tables: offsets (clamped to [0, S]), positions' tokens or slots,
  // routed chunk prefix
  if (tid < 4) s_steps[tid] = 0;
  for (int i = tid; i <= E; i += kWThreads) s_off[i] = min(max(a.offsets[i], 0), a.S);
  for (int i = tid; i < a.S; i += kWThreads)
    s_slots[i] = STAGE == 1 ? a.sorted_slots[i] / a.k : a.sorted_slots[i];
  lds_barrier();
  const int ch0 = a.g[0].ch;
  if (wave == 0) {
    int n[4], tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      n[i] = e < E ? (max(s_off[e + 1] - s_off[e], 0) + ch0 - 1) / ch0 : 0;
      tot += n[i];
    }
    const int incl = wave_inclusive_scan(tot);
    int run = incl - tot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) s_cp[e] = run;
      run += n[i];
    }
    if (lane == kWave - 1) s_cp[E] = incl;
  }
  lds_barrier();
  const int kept = uniform(s_off[E]);

  // ---- stage 2: rows of slot_out whose slots the alignment dropped are zero
  if (STAGE == 2 && a.zero_dropped && kept < a.S) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(bufs);  // free until the first staging
    for (int i = tid; i < (a.S + 31) / 32; i += kWThreads) bits[i] = 0u;
    lds_barrier();
    for (int p = tid; p < kept; p += kWThreads) {
      const int s = s_slots[p];
      if (s >= 0 && s < a.S) atomicOr(bits + (s >> 5), 1u << (s & 31));
    }
    lds_barrier();
    for (int s = b; s < a.S; s += nwg) {
      if ((bits[s >> 5] >> (s & 31)) & 1u) continue;
      for (int c = tid; c < a.H / 4; c += kWThreads)
        gstore<f32x4>(a.slot_out + static_cast<long long>(s) * a.H + 4 * c,
                      f32x4{0.0f, 0.0f, 0.0f, 0.0f});
    }
    lds_barrier();
  }

  // ---- the work list: the shared items first, then the routed experts
  // chunk by chunk, tile by tile.
  // Run-time claims (the usual case): the first Ws workgroups share out the
  // shared items, q each (q shared items about the mean work of a
  // workgroup); every workgroup then claims routed items one by one from a
  // device counter, so the workgroups end together whatever their speed
  // (static ranges of items a few times the mean work would leave some one
  // whole item over it).
  // Static ranges (windows with more items than the workgroups' tables
  // hold): the first Ws workgroups share out the shared items, the others
  // the routed ones, q chosen so that the longer of the two sets is as short
  // as possible (estimated from the items' costs).
  const int n1c = a.shared ? (a.T + a.g[1].ch - 1) / a.g[1].ch : 0;  // shared chunks
  const int nrc = uniform(s_cp[E]);                                  // routed chunks
  const long long n1 = static_cast<long long>(n1c) * a.g[1].tiles;
  const long long n0 = static_cast<long long>(nrc) * a.g[0].tiles;
  const long long c1 = a.g[1].cost, c0 = a.g[0].cost;
  const bool dyn = a.claim != nullptr && n0 > 0 && n1 + n0 <= 16ll * nwg;
  long long Ws = 0;  // workgroups on the shared items
  if (n1 > 0) {
    if (dyn) {
      // (at most 32 static items: the table keeps room for claimed ones)
      const long long q = min(32ll, max(1ll, (n1 * c1 + n0 * c0) / nwg / c1));
      Ws = min((n1 + q - 1) / q, static_cast<long long>(nwg));
    } else if (n0 == 0) {
      Ws = min(n1, static_cast<long long>(nwg));
    } else {
      long long best = -1;
      const long long qa = max(1ll, (n1 * c1 + n0 * c0) / nwg / c1);
      for (long long q = qa; q <= qa + 2; ++q) {
        const long long ws = (n1 + q - 1) / q;
        if (ws >= nwg) continue;
        const long long t = max(q * c1, (n0 * c0 + (nwg - ws) - 1) / (nwg - ws));
        if (best < 0 || t < best) {
          best = t;
          Ws = ws;
        }
      }
    }
  }
  long long lo_l, hi_l;  // the static items
  if (dyn) {
    lo_l = b < Ws ? n1 * b / Ws : 0;
    hi_l = b < Ws ? n1 * (b + 1) / Ws : 0;
  } else if (Ws == 0) {  // one set over the whole list (no shared items, or too few workgroups)
    lo_l = (n1 + n0) * b / nwg;
    hi_l = (n1 + n0) * (b + 1) / nwg;
  } else if (b < Ws) {
    lo_l = n1 * b / Ws;
    hi_l = n1 * (b + 1) / Ws;
  } else {
    const long long wr = nwg - Ws, rb = b - Ws;
    lo_l = n1 + n0 * rb / wr;
    hi_l = n1 + n0 * (rb + 1) / wr;
  }
  const int lo = uniform(static_cast<int>(lo_l));
  const int hi = uniform(static_cast<int>(hi_l));
  if (!dyn && lo >= hi) return;  // the whole workgroup: no barrier follows

  WCtx ctx;
  ctx.bufs = bufs;
  ctx.s_off = s_off;
  ctx.s_cp = s_cp;
  ctx.s_slots = s_slots;
  ctx.ready = s_steps;
  ctx.done = s_steps + 2;
  ctx.n1 = static_cast<int>(n1);
  ctx.n0 = static_cast<int>(n0);
  ctx.nwg = nwg;
  ctx.E = E;
  ctx.T = a.T;
  ctx.wave = wave;
  ctx.lane = lane;
  ctx.lo = lo;
  ctx.ns = hi - lo;
  ctx.dyn = dyn;
  ctx.claim = a.claim;
  ctx.finished = a.finished;
  ctx.items = s_items;
  ctx.ph0 = (a.g[0].nblk + a.g[0].bpp - 1) / a.g[0].bpp;
  ctx.ph1 = (a.g[1].nblk + a.g[1].bpp - 1) / a.g[1].bpp;
  for (int i = tid; i < kWItems; i += kWThreads) {
    if (i < ctx.ns) {
      const It it = decode_item(ctx, lo + i);
      s_items[i] = i32x4{it.e | (it.grp << 16), it.seg0, it.m, it.tile};
    } else {
      s_items[i] = i32x4{kPending, 0, 0, 0};
    }
  }
  lds_barrier();

  if (wave >= kWW) {
    staging_loop<STAGE>(ctx);
    return;
  }
  // streamers: the shared items among the static ones, then the routed ones
  const int ns1 = min(max(static_cast<int>(n1) - lo, 0), ctx.ns);
  int step = 0;
  if (ns1 > 0) stream_pass<kFp16, 128, STAGE, STAGE == 1 ? kNC1 : kNC0, 1, 1>(ctx, 0, ns1, step);
  if (item_valid(ctx, ns1))
    stream_pass<WK, G, STAGE, kNC0, 0, STAGE == 2 ? kSL0 : 1>(ctx, ns1, dyn ? -1 : ctx.ns, step);
}

// ------------------------------------------------------------------ host side

int wide_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int WK, int G, int STAGE>
smoe_status launch_wide(const WArgs& a, long long items, hipStream_t st, const char* who) {
  auto kern = wide_ffn_kernel<WK, G, STAGE>;
  static std::atomic<int> attr_done{0};
  if (!attr_done.load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kWLds) != hipSuccess) {
      set_error("%s: cannot raise the dynamic LDS limit to %d bytes", who, kWLds);
      return SMOE_EHIP;
    }
    attr_done.store(1, std::memory_order_release);
  }
  const int nwg = static_cast<int>(std::max(1ll, std::min<long long>(items, wide_cu_count())));
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(kWThreads), kWLds, st, a);
  return check_launch(who);
}

}  // namespace

// The fp16 h rows, then 256 bytes of the launches' claim counters.
static long long h_rows_bytes(long long T, long long k, long long I, long long Is) {
  return (2 * (T * k * I + T * Is) + 255) / 256 * 256;
}

size_t wide_h_bytes(long long T, long long k, long long I, long long Is) {
  return static_cast<size_t>(h_rows_bytes(T, k, I, Is) + 256);
}

bool wide_applicable(const WideCall& c) {
  const long long S = static_cast<long long>(c.T) * c.k;
  return S >= kWideMinSlots && S <= kWideMaxSlots && c.E <= kMaxE && c.H % 128 == 0 &&
         c.I % 128 == 0 && c.Is % 128 == 0;
}

smoe_status wide_ffn(const WideCall& c, hipStream_t st, const char* who) {
  const long long S = static_cast<long long>(c.T) * c.k;
  const bool shared = c.Is > 0;
  constexpr int kBufBytes = std::max(16 * kNC0 * (2 * kKph0 + kWPad), 16 * kNC1 * (2 * kKph1 + kWPad));
  static_assert(kWTabBytes + 2 * kBufBytes <= kWLds, "two phase buffers and the tables fit the LDS");
  auto base = [&](WArgs& a, int stage) {
    a = WArgs{};
    a.sorted_slots = c.sorted_slots;
    a.offsets = c.offsets;
    a.slot_out = c.slot_out;
    a.E = c.E;
    a.k = c.k;
    a.S = static_cast<int>(S);
    a.T = c.T;
    a.H = c.H;
    a.shared = shared ? 1 : 0;
    a.buf_bytes = kBufBytes;
    a.zero_dropped = stage == 2;
  };
  _Float16* h_r = static_cast<_Float16*>(c.h);
  _Float16* h_s = h_r + S * c.I;
  // claim counters: [0] stage 1 and [1] stage 2 claims, [2], [3] their
  // finish counts; zero in a fresh workspace, and each launch leaves its
  // own at zero
  int* ctr = reinterpret_cast<int*>(static_cast<uint8_t*>(c.h) + h_rows_bytes(c.T, c.k, c.I, c.Is));
  // Work-split cost of a 64-byte block per wave, relative (measured): an
  // INT4 block (dequantised, 64 positions) takes about 2.5x an FP16 block
  // of the 128-token shared chunks, which takes about 1.3x an FP16 block of
  // 64 positions.
  auto block_cost = [](int fmt, int nc) { return fmt == kInt4 ? 10 : (nc > 4 ? 4 : 3); };
  auto fill = [&](WGroup& g, const void* w0, const void* w1, const void* s0, const void* s1,
                  int fmt, int N, int K, int nc, int kph, int sl, const void* src, void* out) {
    g.w[0] = static_cast<const uint8_t*>(w0);
    g.w[1] = static_cast<const uint8_t*>(w1 ? w1 : w0);
    g.s[0] = static_cast<const uint16_t*>(s0);
    g.s[1] = static_cast<const uint16_t*>(s1 ? s1 : s0);
    g.nblk = fmt == kInt4 ? K / 128 : K / 32;
    g.bpp = fmt == kInt4 ? kph / 128 : kph / 32;
    g.slabs = N / 16;
    g.tiles = (g.slabs + kWW * sl - 1) / (kWW * sl);
    g.K = K;
    g.ch = 16 * nc;
    g.kph = kph;
    g.rstride = 2 * kph + kWPad;
    g.w_estride = static_cast<long long>(N) * g.nblk * kBlockBytes;
    g.s_estride = fmt == kInt4 ? static_cast<long long>(N) * (K / c.G) : 0;
    g.cost = static_cast<long long>(g.nblk) * sl * block_cost(fmt, nc);
    g.a = static_cast<const uint16_t*>(src);
    g.out = out;
  };
  // group 0: the routed experts; group 1: the FP16 shared expert
  WArgs a1, a2;
  base(a1, 1);
  base(a2, 2);
  a1.claim = ctr;
  a1.finished = ctr + 2;
  a2.claim = ctr + 1;
  a2.finished = ctr + 3;
  fill(a1.g[0], c.wg, c.wu, c.sg, c.su, c.fmt, c.I, c.H, kNC0, kKph0, 1, c.x, h_r);
  fill(a2.g[0], c.wd, nullptr, c.sd, nullptr, c.fmt, c.H, c.I, kNC0, kKph0, kSL0, h_r,
       c.slot_out);
  if (shared) {
    fill(a1.g[1], c.swg, c.swu, nullptr, nullptr, kFp16, c.Is, c.H, kNC1, kKph1, 1, c.x, h_s);
    fill(a2.g[1], c.swd, nullptr, nullptr, nullptr, kFp16, c.H, c.Is, kNC0, kKph0, 1, h_s,
         c.shared_out);
  } else {
    a1.g[1] = a1.g[0];
    a2.g[1] = a2.g[0];
  }
  // upper bounds of the item counts (routed chunks <= min(E, S) + S / chunk)
  auto items = [&](const WArgs& a) {
    const long long r = (std::min<long long>(c.E, S) + S / a.g[0].ch) * a.g[0].tiles;
    return r + (shared ? (c.T + a.g[1].ch - 1) / a.g[1].ch * static_cast<long long>(a.g[1].tiles)
                       : 0);
  };
  auto launch = [&](int stage) -> smoe_status {
    const WArgs& a = stage == 1 ? a1 : a2;
    const long long n = items(a);
    if (c.fmt == kFp16)
      return stage == 1 ? launch_wide<kFp16, 128, 1>(a, n, st, who)
                        : launch_wide<kFp16, 128, 2>(a, n, st, who);
    switch (c.G) {
      case 32: return stage == 1 ? launch_wide<kInt4, 32, 1>(a, n, st, who)
                                 : launch_wide<kInt4, 32, 2>(a, n, st, who);
      case 64: return stage == 1 ? launch_wide<kInt4, 64, 1>(a, n, st, who)
                                 : launch_wide<kInt4, 64, 2>(a, n, st, who);
      default: return stage == 1 ? launch_wide<kInt4, 128, 1>(a, n, st, who)
                                 : launch_wide<kInt4, 128, 2>(a, n, st, who);
    }
  };
  smoe_status r = launch(1);
  if (r == SMOE_OK) r = launch(2);
  return r;
}

}  // namespace smoe
