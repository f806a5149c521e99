// Short-window expert FFN over tiled weights: the fused multi-expert W4A16
// (or FP16) FFN of a speculative window, for windows of up to 32 tokens.
//
// Specter paper: fused multi-expert draft kernel paragraph (the routed
// tokens are gathered by expert and every active expert's sub-computation
// runs in one launch), expert-wise verification paragraphs (the tokens of an
// expert form one sub-batch whose outputs go back to their slots) and the
// hybrid-precision layout (always-on shared experts stay FP16). Design
// notes, "Streamlined Execution Engine": INT4 weight tiles are dequantised
// inside the GEMM with FP16 activations and FP32 reductions.
//
// Two launches, each over all active routed experts and the optional FP16
// shared expert:
//   stage 1  h[p] = fp16( SiLU(x_t . Wg^T) * (x_t . Wu^T) )   (p = sorted position)
//   stage 2  out[s] = h[p] . Wd^T                             (s = sorted_slots[p])
//
// Layout of a launch: one workgroup per compute unit, eight "streamer" waves
// and one "service" wave.
//  * An item is (chunk of at most 32 positions of one expert, slab of 16
//    output rows), computed over the whole reduction length by the eight
//    streamers together: in stage 1 four of them take the gate rows and four
//    the up rows, and each takes every fourth 64-byte block of k; in stage 2
//    all eight take the down rows, every eighth block. Each streamer adds its
//    blocks into registers (MFMA 16x16x32 f16, activations as A from LDS,
//    weights as B), then leaves its 16 x 16 partial sums in LDS; a barrier
//    ends the item. The service wave adds the partial sums in a fixed order
//    and writes the item's outputs (stage 1: fp16 h; stage 2: fp32 rows).
//    No output is shared between workgroups: no atomics, nothing to clear,
//    the same result on every run.
//  * The streamers never store, so their in-order memory counter holds only
//    weight loads: each keeps a ring of R blocks in flight across items and
//    waits only for the oldest.
//  * Work split: the items (shared expert first, then the routed experts,
//    chunk by chunk, slab by slab) are cut into one contiguous range per
//    workgroup, balanced by the blocks its busiest streamer takes per item
//    plus one per item; computed on the device from the expert offsets, so
//    nothing is read back and no workgroup waits on another.
//  * Activations: at the start each workgroup stages into LDS the rows of
//    every chunk its range touches (stage 1: the x rows of the chunk's
//    tokens; stage 2: the chunk's h rows), 16 bytes of padding per row. If
//    they do not all fit, it stages as many consecutive chunks as fit and
//    stages the next window when its items reach it.
//  * INT4 weights come tiled (smoe_tile_weights): one load of a wave reads a
//    contiguous kilobyte, 16 rows x 64 bytes, the words already in MFMA step
//    order and their nibbles unzipped, so that dequant_word gives natural k
//    order and x needs no permutation. A block's 16 row scales are one
//    contiguous run: lane 16 g + r loads the scale of row r.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "ffn_device.hpp"
#include "ffn_stream.hpp"

namespace smoe {
namespace {

constexpr int kSW = 8;                          // streamer waves
constexpr int kSThreads = (kSW + 1) * kWave;    // + the service wave
constexpr int kSLds = 160 * 1024;               // one workgroup per CU (gfx950)
constexpr int kSPad = 16;                       // bytes of padding per staged row
constexpr int kSNB = 8;                         // staging loads in flight per thread
constexpr int kSMaxSlots = 1024;                // window slots (T*k) the kernel takes
constexpr int kSMaxT = 32;                      // tokens (two MFMA column groups)
#ifndef SMOE_STREAM_RING
#define SMOE_STREAM_RING 8
#endif
constexpr int kRing = SMOE_STREAM_RING;         // weight blocks in flight per streamer

// LDS tables (ints): expert offsets, chunk prefix, sorted slots, then the
// workgroup's range: per chunk (group | expert << 1 | rows << 9, first
// position, arena byte offset, staging window), per item (range chunk |
// slab << 9), per window (first range chunk, staged pieces)
constexpr int kMaxRC = 256;                     // chunks a workgroup's range may touch
constexpr int kMaxItems = 1024;                 // items a workgroup's range may hold
constexpr int kTabOff = 0;
constexpr int kTabCp = kMaxE + 4;
constexpr int kTabSlots = 2 * (kMaxE + 4);
constexpr int kTabChInfo = kTabSlots + kSMaxSlots;
constexpr int kTabChSeg = kTabChInfo + kMaxRC;
constexpr int kTabChOff = kTabChSeg + kMaxRC;
constexpr int kTabChWin = kTabChOff + kMaxRC;
constexpr int kTabItem = kTabChWin + kMaxRC;
constexpr int kTabWinFirst = kTabItem + kMaxItems;
constexpr int kTabWinPieces = kTabWinFirst + kMaxRC + 4;
constexpr int kTabWinItem = kTabWinPieces + kMaxRC + 4;
constexpr int kTabBytes = (kTabWinItem + kMaxRC + 4) * 4;
static_assert(kTabBytes % 16 == 0, "partials must start 16-byte aligned");

struct SGroup {
  const uint8_t* w[2];        // stage 1: gate, up; stage 2: down (w[1] unused)
  const uint16_t* s[2];       // INT4 scales (tiled), null for FP16
  long long w_estride;        // bytes per expert matrix
  long long s_estride;        // scale elements per expert matrix
  int fmt;                    // kInt4 or kFp16
  int nblk;                   // 64-byte blocks per weight row
  int slabs;                  // output rows / 16
  int K;                      // reduction length (elements)
  int csz;                    // positions per chunk
  const uint16_t* a;          // stage 1: x [T][H]; stage 2: this group's h [rows][K]
  void* out;                  // stage 1: h fp16 [rows][N]; stage 2: fp32 [*][H]
  int out_stride;             // elements per output row
};

struct SArgs {
  const int32_t* sorted_slots;
  const int32_t* offsets;
  float* slot_out;            // stage 2: routed output (rows of dropped slots are zeroed)
  int E, k, S, T, H;
  int n_groups;               // 1, or 2 with the shared expert (group 1)
  int arena_off, arena_bytes; // LDS byte range of the staged rows
  SGroup g[2];
};

// Workgroup barrier that orders LDS only. Every barrier of this kernel
// hands over LDS data (tables, staged rows, partial sums); none orders
// global memory, and a full workgroup fence would make each wave wait for
// all of its weight loads in flight first.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A wave-uniform pointer moved to scalar registers (a select between two
// such values stays a select, not a load).
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<P*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// f(integral_constant<int, i>) for i = I .. N-1, unrolled at compile time (the
// register ring needs compile-time slot indices whatever the body's size).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<I + 1, N>(f);
  }
}

// The kernel arguments read in place from the kernel-argument segment.
// Picking a group's field by a run-time index from the by-value argument
// would make the compiler copy the whole argument to scratch memory; a load
// from the constant segment takes the index directly.
typedef const __attribute__((address_space(4))) SArgs ConstArgs;
__device__ __forceinline__ ConstArgs* kargs() {
  return (ConstArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
}
template <int WK, int G, int STAGE, int NC>
__global__ __launch_bounds__(kSThreads, 1) void stream_ffn_kernel(SArgs a) {
  constexpr int NMAT = STAGE == 1 ? 2 : 1;      // matrices per item
  constexpr int WM = kSW / NMAT;                // streamers per matrix
  constexpr int NQ = WK == kInt4 ? 128 / G : 1; // INT4 scales per block and row
  constexpr int NS = NQ == 4 ? 2 : 1;           // scale words per ring entry
  constexpr int PER = G / 32;                   // MFMA steps per INT4 group
  extern __shared__ __align__(16) uint8_t smem[];
  int* tab = reinterpret_cast<int*>(smem);
  int* s_off = tab + kTabOff;
  int* s_cp = tab + kTabCp;
  int* s_slots = tab + kTabSlots;
  int* ch_info = tab + kTabChInfo;
  int* ch_seg = tab + kTabChSeg;
  int* ch_off = tab + kTabChOff;
  int* ch_win = tab + kTabChWin;
  int* it_info = tab + kTabItem;
  int* win_first = tab + kTabWinFirst;
  int* win_pieces = tab + kTabWinPieces;
  int* win_item = tab + kTabWinItem;    // first item of each window, then hi
  f32x4* s_part = reinterpret_cast<f32x4*>(smem + kTabBytes);  // [2][kSW][NC][64]
  uint8_t* arena = smem + a.arena_off;
  ConstArgs* ka = kargs();

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const bool service = wave == kSW;
  const int E = a.E;
  const int b = blockIdx.x;
  const int nwg = gridDim.x;
  // both groups' reduction lengths and activation sources, in scalar
  // registers (the staging loops pick one per lane)
  const int K0 = uniform(a.g[0].K), K1 = uniform(a.g[1].K);
  const uint16_t* src0 = uniform_ptr(a.g[0].a);
  const uint16_t* src1 = uniform_ptr(a.g[1].a);

  // ---- tables: offsets (clamped to [0, S]) and the sorted slots
  for (int i = tid; i <= E; i += kSThreads) s_off[i] = min(max(a.offsets[i], 0), a.S);
  for (int i = tid; i < a.S; i += kSThreads) s_slots[i] = a.sorted_slots[i];
  lds_barrier();
  // chunk prefix over the routed experts (one wave; E <= 256)
  const int csz0 = a.g[0].csz;
  if (wave == 0) {
    int n[4], tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      n[i] = e < E ? (max(s_off[e + 1] - s_off[e], 0) + csz0 - 1) / csz0 : 0;
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

  // ---- stage 2: rows of slot_out whose slots the alignment dropped are
  // zero (every kept slot's row is written by the items)
  if (STAGE == 2 && kept < a.S) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(s_part);  // free until the first item
    for (int i = tid; i < (a.S + 31) / 32; i += kSThreads) bits[i] = 0u;
    lds_barrier();
    for (int p = tid; p < kept; p += kSThreads) {
      const int s = s_slots[p];
      if (s >= 0 && s < a.S) atomicOr(bits + (s >> 5), 1u << (s & 31));
    }
    lds_barrier();
    for (int s = b; s < a.S; s += nwg) {
      if ((bits[s >> 5] >> (s & 31)) & 1u) continue;
      for (int c = tid; c < a.H / 4; c += kSThreads)
        gstore<f32x4>(a.slot_out + static_cast<long long>(s) * a.H + 4 * c,
                      f32x4{0.0f, 0.0f, 0.0f, 0.0f});
    }
    lds_barrier();
  }

  // ---- the work list and this workgroup's range
  const int csz1 = a.g[1].csz;
  const int slabs0 = a.g[0].slabs, slabs1 = a.g[1].slabs;
  const int nblk0 = a.g[0].nblk, nblk1 = a.g[1].nblk;
  const int n1c = a.n_groups > 1 ? (a.T + csz1 - 1) / csz1 : 0;   // shared chunks
  const int nrc = uniform(s_cp[E]);                                  // routed chunks
  const int n1 = n1c * slabs1;
  const long long n0 = static_cast<long long>(nrc) * slabs0;
  const long long c1 = a.n_groups > 1 ? (nblk1 + WM - 1) / WM + 1 : 1;
  const long long c0 = (nblk0 + WM - 1) / WM + 1;
  const long long C = n1 * c1 + n0 * c0;
  auto start_of = [&](long long t) -> long long {  // first item whose cost starts at >= t
    if (t <= n1 * c1) return (t + c1 - 1) / c1;
    return n1 + (t - n1 * c1 + c0 - 1) / c0;
  };
  const int lo = uniform(static_cast<int>(start_of(C * b / nwg)));
  const int hi = uniform(static_cast<int>(start_of(C * (b + 1) / nwg)));
  if (lo >= hi) return;  // the whole workgroup: no barrier follows
  auto gc_of = [&](int item) -> int {
    return item < n1 ? item / slabs1 : n1c + (item - n1) / slabs0;
  };
  const int gc_lo = gc_of(lo);
  const int nch = gc_of(hi - 1) - gc_lo + 1;   // chunks of the range (<= kMaxRC)
  const int nit = hi - lo;                     // items of the range (<= kMaxItems)

  // ---- range tables, built in parallel: chunks, then windows (one thread:
  // consecutive chunks whose rows fit the arena), then items
  for (int t = tid; t < nch; t += kSThreads) {
    const int gc = gc_lo + t;
    int grp, e, seg0, m;
    if (gc < n1c) {
      grp = 1;
      e = 0;
      seg0 = gc * csz1;
      m = min(csz1, a.T - seg0);
    } else {
      const int rc = gc - n1c;
      int lo_e = 0, hi_e = E;  // invariant: s_cp[lo_e] <= rc < s_cp[hi_e]
      while (hi_e - lo_e > 1) {
        const int mid = (lo_e + hi_e) >> 1;
        if (s_cp[mid] <= rc) lo_e = mid; else hi_e = mid;
      }
      grp = 0;
      e = lo_e;
      seg0 = s_off[e] + (rc - s_cp[e]) * csz0;
      m = min(csz0, s_off[e + 1] - seg0);
    }
    ch_info[t] = grp | (e << 1) | (m << 9);
    ch_seg[t] = seg0;
  }
  lds_barrier();
  if (tid == 0) {
    int w = -1, used = 0;
    long long pieces = 0;
    for (int t = 0; t < nch; ++t) {
      const int info = ch_info[t];
      const int grp = info & 1, m = info >> 9;
      const int K = grp ? K1 : K0;
      const int need = m * (2 * K + kSPad);
      if (w < 0 || used + need > a.arena_bytes) {
        if (w >= 0) win_pieces[w] = static_cast<int>(pieces);
        ++w;
        win_first[w] = t;
        used = 0;
        pieces = 0;
      }
      ch_off[t] = used;
      ch_win[t] = w;
      used += need;
      pieces += static_cast<long long>(m) * (K / 8);
    }
    win_pieces[w] = static_cast<int>(pieces);
    win_first[w + 1] = nch;
  }
  for (int t = tid; t < nit; t += kSThreads) {
    const int item = lo + t;
    const int slab = item < n1 ? item % slabs1 : (item - n1) % slabs0;
    it_info[t] = (gc_of(item) - gc_lo) | (slab << 9);
  }
  lds_barrier();
  // first item of each window (windows are consecutive runs of items)
  for (int t = tid; t < nit; t += kSThreads) {
    const int w = ch_win[it_info[t] & 511];
    if (t == 0 || ch_win[it_info[t - 1] & 511] != w) win_item[w] = lo + t;
    if (t == nit - 1) win_item[w + 1] = hi;
  }
  lds_barrier();

  // item -> range chunk, slab, window (wave-uniform)
  auto rc_of = [&](int item) { return uniform(it_info[item - lo] & 511); };
  auto win_of = [&](int item) { return uniform(ch_win[rc_of(item)]); };

  // Stage window w: every thread walks the same number of batches.
  auto stage_window = [&](int w) {
    const int first = uniform(win_first[w]), last = uniform(win_first[w + 1]);
    const int total = uniform(win_pieces[w]);
    const int batches = (total + kSThreads * kSNB - 1) / (kSThreads * kSNB);
    int t = first, base = 0;  // chunk of the current piece, pieces before it
    for (int bt = 0; bt < batches; ++bt) {
      u32x4 v[kSNB];
      int dst[kSNB];
      static_for<0, kSNB>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int q = tid + (bt * kSNB + j) * kSThreads;
        dst[j] = -1;
        if (q < total) {
          int info = ch_info[t];
          int npr = ((info & 1) ? K1 : K0) / 8;
          while (q >= base + (info >> 9) * npr) {
            base += (info >> 9) * npr;
            ++t;
            info = ch_info[t];
            npr = ((info & 1) ? K1 : K0) / 8;
          }
          const int grp = info & 1;
          const int p = q - base;
          const int r = p / npr, c = p - r * npr;
          const int seg0 = ch_seg[t];
          long long row;
          if (STAGE == 1) {
            row = grp == 1 ? seg0 + r : s_slots[seg0 + r] / a.k;  // token
            row = min(max(row, 0ll), static_cast<long long>(a.T - 1));
          } else {
            row = seg0 + r;  // position in the group's h
          }
          const uint16_t* src = grp ? src1 : src0;
          v[j] = gload<u32x4>(src + row * (npr * 8) + 8 * c);
          dst[j] = ch_off[t] + r * (npr * 16 + kSPad) + 16 * c;
        }
      });
      static_for<0, kSNB>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if (dst[j] >= 0) *reinterpret_cast<u32x4*>(arena + dst[j]) = v[j];
      });
    }
    (void)last;
    // every staging load has landed: the loads and LDS writes above are
    // conditional, and the compiler cannot pair them, so without this wait
    // it would carry "load pending" on those registers into the main loop
    // and wait for the weight ring wherever it reuses them
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    lds_barrier();
  };

  if (service) {
    // ---------------------------------------------------------- service wave
    for (int i = lo; i < hi; ++i) {
      if (i == lo || win_of(i) != win_of(i - 1)) stage_window(win_of(i));
      lds_barrier();  // the streamers' partial sums of item i are in LDS
      const int rc = rc_of(i);
      const int info = uniform(ch_info[rc]);
      const int grp = info & 1, m = info >> 9;
      const int seg0 = uniform(ch_seg[rc]);
      const int slab = uniform(it_info[i - lo] >> 9);
      void* out = ka->g[grp].out;
      const long long out_stride = ka->g[grp].out_stride;
      const f32x4* part = s_part + (i & 1) * (kSW * NC * kWave);
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) {
        if (cg > 0 && m <= 16) break;
        f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < kSW; ++w) {
          const f32x4 v = part[(w * NC + cg) * kWave + lane];
          if (STAGE == 1 && w >= WM) s1 += v; else s0 += v;
        }
        const int n = slab * 16 + r16;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int sl = 16 * cg + 4 * g + i4;
          if (sl >= m) continue;
          if (STAGE == 1) {
            const float gv = s0[i4], uv = s1[i4];
            const float h = gv / (1.0f + __expf(-gv)) * uv;
            gstore<_Float16>(static_cast<_Float16*>(out) + (seg0 + sl) * out_stride + n,
                             static_cast<_Float16>(h));
          } else {
            const int row = grp == 1 ? seg0 + sl : s_slots[seg0 + sl];
            if (row < 0 || row >= (grp == 1 ? a.T : a.S)) continue;
            gstore<float>(static_cast<float*>(out) + row * out_stride + n, s0[i4]);
          }
        }
      }
    }
    return;
  }

  // ------------------------------------------------------------ streamers
  const int mm = wave / WM;  // matrix of this wave
  const int kw = wave % WM;  // first block of this wave within a row
  // this wave's matrices and strides of the two groups (scalar registers)
  const uint8_t* w_g0 = ka->g[0].w[mm];
  const uint8_t* w_g1 = ka->g[1].w[mm];
  const uint16_t* s_g0 = ka->g[0].s[mm];
  const uint16_t* s_g1 = ka->g[1].s[mm];
  const long long we0 = a.g[0].w_estride, we1 = a.g[1].w_estride;
  const long long se0 = a.g[0].s_estride, se1 = a.g[1].s_estride;
  const int fmt0 = a.g[0].fmt, fmt1 = a.g[1].fmt;

  struct Cur {  // a position in this wave's block sequence (wave-uniform)
    int item, blk, nblk, fmt, slab;
    const uint8_t* w;
    const uint16_t* s;
  };
  // the first item at or after cu.item in which this wave has blocks
  auto settle = [&](Cur& cu) {
    if (cu.item < n1 && kw >= nblk1) cu.item = n1;
    if (cu.item >= n1 && kw >= nblk0) cu.item = hi;
    if (cu.item < hi) {
      const int rc = rc_of(cu.item);
      const int info = uniform(ch_info[rc]);
      const int grp = info & 1, e = (info >> 1) & 255;
      cu.slab = uniform(it_info[cu.item - lo] >> 9);
      cu.nblk = grp ? nblk1 : nblk0;
      cu.fmt = grp ? fmt1 : fmt0;
      cu.w = (grp ? w_g1 : w_g0) + e * (grp ? we1 : we0);
      cu.s = (grp ? s_g1 : s_g0) + e * (grp ? se1 : se0);
      cu.blk = kw;
    }
  };

  // (NQ = 1: the scale is kept as loaded, 16 bits, with no masking to
  // place: a mask applied after the load was hoisted to the loop's back
  // edge, where it waited for every load in flight)
  struct Entry {
    u32x4 v;
    uint32_t s[NS];
    uint16_t s16;
  };
  Entry ring[kRing];
  // Every slot of the ring takes a load on every pass, also past the end of
  // the sequence (the last block again), and INT4 launches load a scale for
  // FP16 blocks too (from the block itself): with the same loads on every
  // path the compiler waits only for the oldest block, not for all of them.
  auto load = [&](Entry& en, const Cur& cu) {
    const long long tb =
        static_cast<long long>(cu.slab) * cu.nblk + min(cu.blk, cu.nblk - 1);  // tile block
    en.v = gload<u32x4>(cu.w + tb * 1024 + 16 * lane);
    if (WK == kInt4) {
      const uint16_t* sp = cu.fmt == kInt4
                               ? cu.s + (tb * 16 + r16) * NQ
                               : reinterpret_cast<const uint16_t*>(cu.w + tb * 1024 + 16 * lane);
      if (NQ == 1) {
        en.s16 = gload<uint16_t>(sp);
      } else if (NQ == 2) {
        en.s[0] = gload<uint32_t>(sp);
      } else {
        const u32x2 v2 = gload<u32x2>(sp);
        en.s[0] = v2[0];
        en.s[NS - 1] = v2[1];
      }
    }
  };

  f32x4 acc[NC];
#pragma unroll
  for (int cg = 0; cg < NC; ++cg) acc[cg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t dq_lo = 0x000F000Fu, dq_hi = 0x00F000F0u, dq_magic = 0x64006400u;
  asm volatile("" : "+v"(dq_lo), "+v"(dq_hi), "+v"(dq_magic));  // keep the masks in VGPRs

  // A-operand rows of the compute item (LDS byte offsets; -1: past the chunk)
  int arow[NC];
  int cm = 0;  // positions of the compute item's chunk
  auto set_rows = [&](int item) {
    const int rc = rc_of(item);
    const int info = uniform(ch_info[rc]);
    const int grp = info & 1;
    cm = info >> 9;
    const int off = uniform(ch_off[rc]);
    const int st = 2 * (grp ? K1 : K0) + kSPad;
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
      const int r = 16 * cg + r16;
      arow[cg] = r < cm ? off + r * st : -1;
    }
  };
  // end of item i: partial sums to LDS and the item's barrier
  auto item_end = [&](int i) {
    f32x4* part = s_part + (i & 1) * (kSW * NC * kWave);
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
      part[(wave * NC + cg) * kWave + lane] = acc[cg];
      acc[cg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    lds_barrier();
  };
  auto lds16 = [&](int off) -> f16x8 {
    return *reinterpret_cast<const f16x8*>(arena + off);
  };
  auto compute = [&](const Entry& en, const Cur& cu) {
    const bool wide = NC > 1 && cm > 16;
    if (WK == kInt4 && cu.fmt == kInt4) {
      const int kk = cu.blk * 128;
      f16x8 B[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) B[q] = dequant_word(en.v[q], dq_lo, dq_hi, dq_magic);
#pragma unroll
      for (int gq = 0; gq < NQ; ++gq) {
        uint16_t sbits;
        if (NQ == 1) {
          sbits = en.s16;
        } else {
          const uint32_t word = en.s[NQ == 4 ? (gq >> 1) : 0];
          sbits = static_cast<uint16_t>((gq & 1) ? (word >> 16) : word);
        }
        const float sc = static_cast<float>(bitcast<_Float16>(sbits));
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) {
          if (cg > 0 && !wide) break;
          f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int qq = 0; qq < PER; ++qq) {
            const int q = gq * PER + qq;
            f16x8 A = {};
            if (arow[cg] >= 0) A = lds16(arow[cg] + 2 * (kk + 8 * int4_word(G, g, q)));
            t = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[q], t, 0, 0, 0);
          }
          acc[cg] += sc * t;
        }
      }
    } else {
      const int kk = cu.blk * 32;
      const f16x8 B = bitcast<f16x8>(en.v);
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) {
        if (cg > 0 && !wide) break;
        f16x8 A = {};
        if (arow[cg] >= 0) A = lds16(arow[cg] + 2 * (kk + 8 * g));
        acc[cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc[cg], 0, 0, 0);
      }
    }
  };

  // The range in segments, one per staging window: stage the window while
  // the ring's first loads are in flight, then full passes over the ring
  // (compute a slot, load the slot R blocks ahead; past the segment's end
  // the loads repeat its last block), then the last blocks without loads.
  // Item ends come before the first block of the next item. The pass loop
  // is entered only with a full ring, so the compiler waits for the oldest
  // block alone.
  auto per_item = [&](int nb) { return kw < nb ? (nb - kw + WM - 1) / WM : 0; };
  int cur = lo;  // first item whose end is not processed yet
  for (int w = 0;; ++w) {
    const int seg_lo = uniform(win_item[w]), seg_hi = uniform(win_item[w + 1]);
    Cur L;
    L.item = seg_lo;
    L.blk = 0;
    L.nblk = 1;
    L.fmt = fmt0;
    L.slab = 0;
    L.w = w_g0;  // (a wave without blocks in the segment still loads, in bounds)
    L.s = s_g0;
    auto settle_seg = [&](Cur& cu) {
      settle(cu);
      if (cu.item > seg_hi) cu.item = seg_hi;
    };
    auto advance_seg = [&](Cur& cu) {
      cu.blk += WM;
      if (cu.blk >= cu.nblk && cu.item < seg_hi) {
        ++cu.item;
        if (cu.item < seg_hi) settle_seg(cu);
      }
    };
    settle_seg(L);
    Cur Cc = L;
    static_for<0, kRing>([&](auto rc) {
      load(ring[decltype(rc)::value], L);
      advance_seg(L);
    });
    stage_window(w);
    const int i1 = min(seg_hi, n1) - min(seg_lo, n1);
    int left = i1 * per_item(nblk1) + (seg_hi - seg_lo - i1) * per_item(nblk0);
    int rows_item = -1;  // item whose A rows arow[] describe
    while (left >= kRing) {
#pragma clang loop unroll(full)
      for (int r = 0; r < kRing; ++r) {
        if (Cc.item != rows_item) {
          while (cur < Cc.item) {  // ends of the items before it
            item_end(cur);
            ++cur;
          }
          set_rows(Cc.item);
          rows_item = Cc.item;
        }
        compute(ring[r], Cc);
        load(ring[r], L);
        advance_seg(L);
        advance_seg(Cc);
      }
      left -= kRing;
    }
#pragma clang loop unroll(full)
    for (int r = 0; r < kRing; ++r) {
      if (r < left) {
        if (Cc.item != rows_item) {
          while (cur < Cc.item) {
            item_end(cur);
            ++cur;
          }
          set_rows(Cc.item);
          rows_item = Cc.item;
        }
        compute(ring[r], Cc);
        advance_seg(Cc);
      }
    }
    while (cur < seg_hi) {
      item_end(cur);
      ++cur;
    }
    if (seg_hi >= hi) break;
  }
}

// ------------------------------------------------------------------ host side

int stream_cu_count() {
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

constexpr int kPartBytesPerNc = 2 * kSW * kWave * 16;  // double-buffered partials per column group

int arena_bytes(int nc) { return kSLds - kTabBytes - nc * kPartBytesPerNc; }

template <int WK, int G, int STAGE, int NC>
smoe_status launch_stream(const SArgs& a, long long items, hipStream_t st, const char* who) {
  auto kern = stream_ffn_kernel<WK, G, STAGE, NC>;
  static std::atomic<int> attr_done{0};
  if (!attr_done.load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kSLds) != hipSuccess) {
      set_error("%s: cannot raise the dynamic LDS limit to %d bytes", who, kSLds);
      return SMOE_EHIP;
    }
    attr_done.store(1, std::memory_order_release);
  }
  const int nwg = static_cast<int>(std::max(1ll, std::min<long long>(items, stream_cu_count())));
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(kSThreads), kSLds, st, a);
  return check_launch(who);
}

// Upper bound of the items (and so of the chunks) one workgroup's range can
// hold, for a work list of at most `items0` routed and `items1` shared items
// over `nwg` workgroups: the range spans the cost C / nwg, rounded up by one
// item at each end.
long long range_items_bound(long long items0, long long c0, long long items1, long long c1,
                            int nwg) {
  const long long C = items0 * c0 + items1 * c1;
  const long long cmin = std::max(1ll, std::min(c0, items1 > 0 ? c1 : c0));
  const long long cmax = std::max(c0, items1 > 0 ? c1 : c0);
  return (C / std::max(1, nwg) + 2 * cmax) / cmin + 2;
}

template <int WK, int G>
smoe_status launch_pair(const SArgs& a1, int nc1, long long items1, const SArgs& a2, int nc2,
                        long long items2, hipStream_t st, const char* who) {
  smoe_status s = nc1 == 2 ? launch_stream<WK, G, 1, 2>(a1, items1, st, who)
                           : launch_stream<WK, G, 1, 1>(a1, items1, st, who);
  if (s != SMOE_OK) return s;
  return nc2 == 2 ? launch_stream<WK, G, 2, 2>(a2, items2, st, who)
                  : launch_stream<WK, G, 2, 1>(a2, items2, st, who);
}

}  // namespace

size_t stream_h_bytes(long long T, long long k, long long I, long long Is) {
  const long long bytes = 2 * (T * k * I + T * Is);
  return static_cast<size_t>((bytes + 255) / 256 * 256);
}

smoe_status stream_ffn(const StreamCall& c, hipStream_t st, const char* who) {
  const long long S = static_cast<long long>(c.T) * c.k;
  if (c.T <= 0 || c.T > kSMaxT || S > kSMaxSlots || c.E > kMaxE) return kStreamNotApplicable;
  const bool shared = c.Is > 0;
  const int nbytes_k = c.fmt == kInt4 ? 1 : 4;  // 2 * bytes per k: INT4 1/2 B, FP16 2 B
  (void)nbytes_k;
  // routed chunks: up to 16 positions, 32 when an expert is likely to hold
  // more than 16 of the window's slots; the shared expert takes the window
  // in one chunk (every token)
  const int csz_r = (c.T > 16 && (c.T > 24 || S > 8 * std::min<long long>(c.E, S)))
                        ? std::min(c.T, 32) : std::min(c.T, 16);
  const int csz_s = c.T;
  auto fit = [&](int csz, int K, int nc) {  // positions whose rows fit the arena
    return std::min(csz, arena_bytes(nc) / (2 * K + kSPad));
  };
  // stage 1 reads x rows (K = H), stage 2 h rows (K = I or Is)
  int nc1 = std::max(csz_r, shared ? csz_s : 0) > 16 ? 2 : 1;
  int r1 = fit(csz_r, c.H, nc1), s1 = shared ? fit(csz_s, c.H, nc1) : 1;
  int nc2 = nc1;
  int r2 = fit(csz_r, c.I, nc2), s2 = shared ? fit(csz_s, c.Is, nc2) : 1;
  if (r1 < 1 || s1 < 1 || r2 < 1 || s2 < 1) return kStreamNotApplicable;
  if (std::max(r1, shared ? s1 : 0) <= 16) nc1 = 1;
  if (std::max(r2, shared ? s2 : 0) <= 16) nc2 = 1;

  SArgs a1{}, a2{};
  for (SArgs* a : {&a1, &a2}) {
    a->sorted_slots = c.sorted_slots;
    a->offsets = c.offsets;
    a->slot_out = c.slot_out;
    a->E = c.E;
    a->k = c.k;
    a->S = static_cast<int>(S);
    a->T = c.T;
    a->H = c.H;
    a->n_groups = shared ? 2 : 1;
    a->arena_off = kTabBytes + (a == &a1 ? nc1 : nc2) * kPartBytesPerNc;
    a->arena_bytes = arena_bytes(a == &a1 ? nc1 : nc2);
  }
  _Float16* h_r = static_cast<_Float16*>(c.h);
  _Float16* h_s = h_r + S * c.I;
  const int row_i4 = c.fmt == kInt4 ? 1 : 0;
  // stage 1: gate and up, [E][I][H]
  {
    SGroup& g = a1.g[0];
    g.w[0] = static_cast<const uint8_t*>(c.wg);
    g.w[1] = static_cast<const uint8_t*>(c.wu);
    g.s[0] = static_cast<const uint16_t*>(c.sg);
    g.s[1] = static_cast<const uint16_t*>(c.su);
    g.fmt = c.fmt;
    g.K = c.H;
    g.nblk = row_i4 ? c.H / 128 : c.H / 32;
    g.slabs = c.I / 16;
    g.w_estride = static_cast<long long>(c.I) * g.nblk * kBlockBytes;
    g.s_estride = row_i4 ? static_cast<long long>(c.I) * (c.H / c.G) : 0;
    g.csz = r1;
    g.a = static_cast<const uint16_t*>(c.x);
    g.out = h_r;
    g.out_stride = c.I;
  }
  // stage 2: down, [E][H][I]
  {
    SGroup& g = a2.g[0];
    g.w[0] = g.w[1] = static_cast<const uint8_t*>(c.wd);
    g.s[0] = g.s[1] = static_cast<const uint16_t*>(c.sd);
    g.fmt = c.fmt;
    g.K = c.I;
    g.nblk = row_i4 ? c.I / 128 : c.I / 32;
    g.slabs = c.H / 16;
    g.w_estride = static_cast<long long>(c.H) * g.nblk * kBlockBytes;
    g.s_estride = row_i4 ? static_cast<long long>(c.H) * (c.I / c.G) : 0;
    g.csz = r2;
    g.a = reinterpret_cast<const uint16_t*>(h_r);
    g.out = c.slot_out;
    g.out_stride = c.H;
  }
  if (shared) {
    SGroup& g1 = a1.g[1];
    g1.w[0] = static_cast<const uint8_t*>(c.swg);
    g1.w[1] = static_cast<const uint8_t*>(c.swu);
    g1.s[0] = g1.s[1] = nullptr;
    g1.fmt = kFp16;
    g1.K = c.H;
    g1.nblk = c.H / 32;
    g1.slabs = c.Is / 16;
    g1.w_estride = 0;
    g1.s_estride = 0;
    g1.csz = s1;
    g1.a = static_cast<const uint16_t*>(c.x);
    g1.out = h_s;
    g1.out_stride = c.Is;
    SGroup& g2 = a2.g[1];
    g2.w[0] = g2.w[1] = static_cast<const uint8_t*>(c.swd);
    g2.s[0] = g2.s[1] = nullptr;
    g2.fmt = kFp16;
    g2.K = c.Is;
    g2.nblk = c.Is / 32;
    g2.slabs = c.H / 16;
    g2.w_estride = 0;
    g2.s_estride = 0;
    g2.csz = s2;
    g2.a = reinterpret_cast<const uint16_t*>(h_s);
    g2.out = c.shared_out;
    g2.out_stride = c.H;
  } else {
    a1.g[1] = a1.g[0];
    a2.g[1] = a2.g[0];
    a1.g[1].csz = a2.g[1].csz = 1;
  }
  // upper bounds of the item counts (routed chunks <= min(E, S) + S / csz)
  auto items = [&](const SArgs& a) {
    const long long rc = std::min<long long>(c.E, S) + S / a.g[0].csz;
    long long n = rc * a.g[0].slabs;
    if (shared) n += (c.T + a.g[1].csz - 1) / a.g[1].csz * static_cast<long long>(a.g[1].slabs);
    return n;
  };
  const long long items1 = items(a1), items2 = items(a2);
  // every range must fit the LDS tables (chunks and items of a workgroup)
  for (const SArgs* a : {&a1, &a2}) {
    const int wm = a == &a1 ? kSW / 2 : kSW;
    const long long i1 = shared ? (c.T + a->g[1].csz - 1) / a->g[1].csz *
                                      static_cast<long long>(a->g[1].slabs) : 0;
    const long long i0 = (a == &a1 ? items1 : items2) - i1;
    const int nwg = static_cast<int>(std::min<long long>(a == &a1 ? items1 : items2,
                                                         stream_cu_count()));
    const long long bound = range_items_bound(i0, (a->g[0].nblk + wm - 1) / wm + 1, i1,
                                              (a->g[1].nblk + wm - 1) / wm + 1, nwg);
    if (bound > std::min(kMaxRC, kMaxItems)) return kStreamNotApplicable;
  }
  if (c.fmt == kFp16) return launch_pair<kFp16, 128>(a1, nc1, items1, a2, nc2, items2, st, who);
  switch (c.G) {
    case 32: return launch_pair<kInt4, 32>(a1, nc1, items1, a2, nc2, items2, st, who);
    case 64: return launch_pair<kInt4, 64>(a1, nc1, items1, a2, nc2, items2, st, who);
    default: return launch_pair<kInt4, 128>(a1, nc1, items1, a2, nc2, items2, st, who);
  }
}

}  // namespace smoe
