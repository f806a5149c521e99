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
// k-phase (double-buffered, one barrier per phase), while the eight stream
// their weight rows through a register ring of R blocks that runs on across
// phases and items (the streamers never wait on anything but their oldest
// weight block and the phase barrier). INT4 and FP16 weights come tiled
// (smoe_tile_weights): one wave load reads 16 rows x 64 bytes in one piece.
//
// Work split: the items (shared expert first, then the routed experts chunk
// by chunk, tile by tile) are cut into one contiguous range per workgroup,
// balanced by the weight blocks a wave streams per item; computed on the
// device from the expert offsets, nothing read back.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "ffn_device.hpp"
#include "ffn_wide.hpp"

namespace smoe {
namespace {

constexpr int kWW = 8;                        // streamer waves
#ifndef SMOE_WIDE_STAGERS
#define SMOE_WIDE_STAGERS 4
#endif
constexpr int kWS = SMOE_WIDE_STAGERS;        // staging waves
constexpr int kWThreads = (kWW + kWS) * kWave;
constexpr int kWLds = 160 * 1024;             // one workgroup per CU (gfx950)
constexpr int kWPad = 16;                     // bytes of padding per staged row
#ifndef SMOE_WIDE_NB
#define SMOE_WIDE_NB 16
#endif
constexpr int kWStageNB = SMOE_WIDE_NB;       // staging loads in flight per lane
#ifndef SMOE_WIDE_RING
#define SMOE_WIDE_RING 4
#endif
constexpr int kWRing = SMOE_WIDE_RING;        // weight blocks in flight per streamer
constexpr int kWTabInts = 2 * (kMaxE + 4) + kWideMaxSlots;
constexpr int kWTabBytes = (kWTabInts * 4 + 15) / 16 * 16;

struct WGroup {
  const uint8_t* w[2];      // stage 1: gate, up; stage 2: down (w[1] = w[0])
  const uint16_t* s[2];     // INT4 scales (tiled), null for FP16
  long long w_estride;      // bytes per expert matrix
  long long s_estride;      // scale elements per expert matrix
  int fmt;                  // kInt4 or kFp16
  int nblk;                 // 64-byte blocks per weight row
  int bpp;                  // blocks per staged k-phase
  int slabs;                // output rows / 16
  int tiles;                // ceil(slabs / 8)
  int K;                    // reduction length (elements)
  int ch;                   // positions per chunk
  const uint16_t* a;        // stage 1: x [T][H]; stage 2: this group's h [rows][K]
  void* out;                // stage 1: fp16 h [rows][N]; stage 2: fp32 [*][H]
  int rows;                 // positions of the group (S routed, T shared)
};

struct WArgs {
  const int32_t* sorted_slots;
  const int32_t* offsets;
  float* slot_out;          // stage 2: rows of dropped slots are zeroed
  int E, k, S, T, H;
  int n_groups;             // 1, or 2 with the shared expert (group 1)
  int kph;                  // k per staged phase (elements)
  int rstride;              // LDS bytes per staged row
  int buf_bytes;            // LDS bytes per phase buffer
  int zero_dropped;         // stage 2: zero the slot_out rows of dropped slots
  WGroup g[2];
};

typedef const __attribute__((address_space(4))) WArgs ConstWArgs;
__device__ __forceinline__ ConstWArgs* wkargs() {
  return (ConstWArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
}

// Workgroup barrier that orders LDS only: every barrier here hands over LDS
// data (tables, staged rows); a full fence would wait for the weight loads
// in flight too.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

template <int WK, int G, int STAGE, int NC>
__global__ __launch_bounds__(kWThreads, 1) void wide_ffn_kernel(WArgs a) {
  constexpr int NMAT = STAGE == 1 ? 2 : 1;
  constexpr int NQ = WK == kInt4 ? 128 / G : 1;  // INT4 scales per block and row
  constexpr int NS = NQ == 4 ? 2 : 1;
  constexpr int PER = G / 32;                    // MFMA steps per INT4 group
  constexpr int CH = 16 * NC;
  extern __shared__ __align__(16) uint8_t smem[];
  int* s_off = reinterpret_cast<int*>(smem);
  int* s_cp = s_off + kMaxE + 4;
  int* s_slots = s_off + 2 * (kMaxE + 4);
  uint8_t* bufs = smem + kWTabBytes;
  ConstWArgs* ka = wkargs();

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int E = a.E;
  const int b = blockIdx.x;
  const int nwg = gridDim.x;

  // ---- tables: offsets (clamped to [0, S]), sorted slots, chunk prefix
  for (int i = tid; i <= E; i += kWThreads) s_off[i] = min(max(a.offsets[i], 0), a.S);
  for (int i = tid; i < a.S; i += kWThreads) s_slots[i] = a.sorted_slots[i];
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

  // ---- the work list and this workgroup's range
  const int ch1 = a.g[1].ch;
  const int tiles0 = a.g[0].tiles, tiles1 = a.g[1].tiles;
  const int nblk0 = a.g[0].nblk, nblk1 = a.g[1].nblk;
  const int bpp0 = a.g[0].bpp, bpp1 = a.g[1].bpp;
  const int n1c = a.n_groups > 1 ? (a.T + ch1 - 1) / ch1 : 0;  // shared chunks
  const int nrc = uniform(s_cp[E]);                               // routed chunks
  const long long n1 = static_cast<long long>(n1c) * tiles1;
  const long long n0 = static_cast<long long>(nrc) * tiles0;
  const long long c1 = a.n_groups > 1 ? nblk1 : 1;
  const long long c0 = nblk0;
  const long long C = n1 * c1 + n0 * c0;
  auto start_of = [&](long long t) -> long long {  // first item whose cost starts at >= t
    if (t <= n1 * c1) return (t + c1 - 1) / c1;
    return n1 + (t - n1 * c1 + c0 - 1) / c0;
  };
  const int lo = uniform(static_cast<int>(start_of(C * b / nwg)));
  const int hi = uniform(static_cast<int>(start_of(C * (b + 1) / nwg)));
  if (lo >= hi) return;  // the whole workgroup: no barrier follows

  // item -> (group, expert, first position, positions, tile); wave-uniform
  struct It {
    int grp, e, seg0, m, tile;
  };
  auto decode = [&](int item) __attribute__((always_inline)) {
    It it;
    if (item < n1) {
      const int c = item / tiles1;
      it.grp = 1;
      it.e = 0;
      it.tile = item - c * tiles1;
      it.seg0 = c * ch1;
      it.m = min(ch1, a.T - it.seg0);
    } else {
      const int ri = item - static_cast<int>(n1);
      const int rc = ri / tiles0;
      it.grp = 0;
      it.tile = ri - rc * tiles0;
      int lo_e = 0, hi_e = E;  // s_cp[lo_e] <= rc < s_cp[hi_e]
      while (hi_e - lo_e > 1) {
        const int mid = (lo_e + hi_e) >> 1;
        if (s_cp[mid] <= rc) lo_e = mid; else hi_e = mid;
      }
      it.e = lo_e;
      it.seg0 = s_off[lo_e] + (rc - s_cp[lo_e]) * ch0;
      it.m = min(ch0, s_off[lo_e + 1] - it.seg0);
    }
    it.grp = uniform(it.grp);
    it.e = uniform(it.e);
    it.seg0 = uniform(it.seg0);
    it.m = uniform(it.m);
    it.tile = uniform(it.tile);
    return it;
  };
  // phases of an item's group
  auto phases_of = [&](int grp) __attribute__((always_inline)) { return grp ? (nblk1 + bpp1 - 1) / bpp1 : (nblk0 + bpp0 - 1) / bpp0; };

  const int K0 = uniform(a.g[0].K), K1 = uniform(a.g[1].K);
  const uint16_t* src0 = uniform_ptr(a.g[0].a);
  const uint16_t* src1 = uniform_ptr(a.g[1].a);

  if (wave >= kWW) {
    // ------------------------------------------------------------ staging waves
    const int sl = (wave - kWW) * kWave + lane;  // this lane among the staging lanes
    // stage (item, phase) into buffer `buf`: rows [0, m), k [p*kph, ...)
    auto stage = [&](const It& it, int p, int buf) __attribute__((always_inline)) {
      const int K = it.grp ? K1 : K0;
      const int k0 = p * a.kph;
      const int kl = min(a.kph, K - k0);
      const int npr = kl / 8;  // 16-byte pieces per row
      const int tot = it.m * npr;
      const uint16_t* src = it.grp ? src1 : src0;
      uint8_t* dst0 = bufs + buf * a.buf_bytes;
      for (int base = 0; base < tot; base += kWS * kWave * kWStageNB) {
        u32x4 v[kWStageNB];
        int dst[kWStageNB];
        static_for<0, kWStageNB>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          const int q = base + j * (kWS * kWave) + sl;
          const int qc = min(q, tot - 1);
          const int r = qc / npr, c = qc - r * npr;
          long long row;
          if (STAGE == 1) {
            row = it.grp ? it.seg0 + r : s_slots[it.seg0 + r] / a.k;  // token
            row = min(max(row, 0ll), static_cast<long long>(a.T - 1));
          } else {
            row = it.seg0 + r;  // position in the group's h
          }
          v[j] = gload<u32x4>(src + row * K + k0 + 8 * c);
          dst[j] = q < tot ? r * a.rstride + 16 * c : -1;
        });
        static_for<0, kWStageNB>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          if (dst[j] >= 0) *reinterpret_cast<u32x4*>(dst0 + dst[j]) = v[j];
        });
      }
    };
    int step = 0;
    It it = decode(lo);
    int p = 0;
    stage(it, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the rows are in LDS
    for (int item = lo;;) {
      lds_barrier();  // B_step: step staged, the buffer of step - 1 is free
      // the next step: next phase of this item, or the next item's first
      int nitem = item, np = p + 1;
      if (np >= phases_of(it.grp)) {
        ++nitem;
        np = 0;
      }
      if (nitem >= hi) break;
      const It nit = nitem == item ? it : decode(nitem);
      stage(nit, np, (step + 1) & 1);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      item = nitem;
      p = np;
      it = nit;
      ++step;
    }
    return;
  }

  // ------------------------------------------------------------ streamers
  // this wave's 16 rows of each item's tile: slab tile * 8 + wave
  const uint8_t* w_g0[2] = {ka->g[0].w[0], ka->g[0].w[1]};
  const uint8_t* w_g1[2] = {ka->g[1].w[0], ka->g[1].w[1]};
  const uint16_t* s_g0[2] = {ka->g[0].s[0], ka->g[0].s[1]};
  const long long we0 = a.g[0].w_estride, we1 = a.g[1].w_estride;
  const long long se0 = a.g[0].s_estride;
  const int fmt0 = a.g[0].fmt;
  const int slabs0 = a.g[0].slabs, slabs1 = a.g[1].slabs;

  struct Cur {  // a position in the wave's block sequence (wave-uniform)
    int item, blk, nblk, bpp, fmt;
    const uint8_t* w[2];
    const uint16_t* s;
    long long tb0;  // first tile block of the wave's slab
  };
  auto settle = [&](Cur& cu) __attribute__((always_inline)) {  // at the start of item cu.item (< hi)
    const It it = decode(cu.item);
    const int grp = it.grp;
    const int slabs = grp ? slabs1 : slabs0;
    const int slab = min(it.tile * kWW + wave, slabs - 1);  // (past N: loaded, never stored)
    cu.nblk = grp ? nblk1 : nblk0;
    cu.bpp = grp ? bpp1 : bpp0;
    cu.fmt = grp ? kFp16 : fmt0;
    cu.tb0 = static_cast<long long>(slab) * cu.nblk;
#pragma unroll
    for (int m = 0; m < 2; ++m)
      cu.w[m] = grp ? w_g1[m] : w_g0[m] + it.e * we0;
    (void)we1;
    cu.s = grp ? nullptr : s_g0[0] + it.e * se0;
    cu.blk = 0;
  };

  struct Entry {
    u32x4 v[NMAT];
    uint32_t s[NMAT][NS];
    uint16_t s16[NMAT];
  };
  constexpr int R = kWRing / NMAT;  // ring entries: kWRing weight blocks in flight
  Entry ring[R];
  const long long s_mstride = WK == kInt4 ? reinterpret_cast<const uint16_t*>(ka->g[0].s[1]) -
                                                reinterpret_cast<const uint16_t*>(ka->g[0].s[0])
                                          : 0;
  // Every ring slot takes a load on every pass, also past the end of the
  // range (the last block again), and INT4 launches load a scale for FP16
  // blocks too (from the block itself), so that the compiler waits only for
  // the oldest block.
  auto load = [&](Entry& en, const Cur& cu) __attribute__((always_inline)) {
    const long long tb = cu.tb0 + min(cu.blk, cu.nblk - 1);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      en.v[m] = gload<u32x4>(cu.w[m] + tb * 1024 + 16 * lane);
      if (WK == kInt4) {
        const uint16_t* sp = cu.fmt == kInt4
                                 ? cu.s + m * s_mstride + (tb * 16 + r16) * NQ
                                 : reinterpret_cast<const uint16_t*>(cu.w[m] + tb * 1024 + 16 * lane);
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
  auto advance = [&](Cur& cu) __attribute__((always_inline)) {
    if (++cu.blk >= cu.nblk && cu.item < hi) {
      ++cu.item;
      if (cu.item < hi) settle(cu);
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
  int cur_m = 0, step = 0;
  It cit;        // the item being computed
  auto set_rows = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
      const int r = min(16 * cg + r16, max(cur_m - 1, 0));
      arow[cg] = buf * a.buf_bytes + r * a.rstride;
    }
  };
  auto lds16 = [&](int off) __attribute__((always_inline)) -> f16x8 {
    return *reinterpret_cast<const f16x8*>(bufs + off);
  };
  // one block at k offset kk within the phase
  auto compute = [&](const Entry& en, const Cur& cu, int kk) __attribute__((always_inline)) {
    // Every column group is computed, also past the chunk's positions (their
    // rows repeat the last staged one and are never stored): with a run-time
    // skip per column group between the MFMAs, the g32 kernels gave wrong
    // rows at a ring depth of four blocks, and without the branches they do
    // not.
    if (WK == kInt4 && cu.fmt == kInt4) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        f16x8 B[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) B[q] = dequant_word(en.v[m][q], dq_lo, dq_hi, dq_magic);
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) {
          uint16_t sbits;
          if (NQ == 1) {
            sbits = en.s16[m];
          } else {
            const uint32_t word = en.s[m][NQ == 4 ? (gq >> 1) : 0];
            sbits = static_cast<uint16_t>((gq & 1) ? (word >> 16) : word);
          }
          const float sc = static_cast<float>(bitcast<_Float16>(sbits));
#pragma unroll
          for (int cg = 0; cg < NC; ++cg) {
            f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int qq = 0; qq < PER; ++qq) {
              const int q = gq * PER + qq;
              const f16x8 A = lds16(arow[cg] + 2 * (kk + 8 * int4_word(G, g, q)));
              t = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[q], t, 0, 0, 0);
            }
            acc[m][cg] += sc * t;
            // one column group's operands in registers at a time
            if (NC > 4) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else {
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) {
        const f16x8 A = lds16(arow[cg] + 2 * (kk + 8 * g));
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
          acc[m][cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bitcast<f16x8>(en.v[m]),
                                                              acc[m][cg], 0, 0, 0);
        if (NC > 4) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // outputs of the finished item cit, then the accumulators back to zero
  auto item_end = [&]() __attribute__((always_inline)) {
    const int grp = cit.grp;
    const int slabs = grp ? slabs1 : slabs0;
    const int slab = cit.tile * kWW + wave;
    if (slab < slabs) {
      const int n = slab * 16 + r16;
      void* out = ka->g[grp].out;
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * cg + 4 * g + i;
          if (r >= cit.m) continue;
          if (STAGE == 1) {
            const int N = slabs * 16;
            const float gv = acc[0][cg][i], uv = acc[NMAT - 1][cg][i];
            const float h = gv / (1.0f + __expf(-gv)) * uv;
            gstore<_Float16>(static_cast<_Float16*>(out) +
                                 static_cast<long long>(cit.seg0 + r) * N + n,
                             static_cast<_Float16>(h));
          } else {
            const int row = grp ? cit.seg0 + r : s_slots[cit.seg0 + r];
            if (row < 0 || row >= (grp ? a.T : a.S)) continue;
            gstore<float>(static_cast<float*>(out) + static_cast<long long>(row) * a.H + n,
                          acc[0][cg][i]);
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
  auto begin_step = [&](const Cur& cu) __attribute__((always_inline)) {
    if (cu.blk == 0) {
      if (cu.item != lo) item_end();
      cit = decode(cu.item);
      cur_m = cit.m;
    }
    lds_barrier();
    set_rows(step & 1);
    ++step;
  };

  // total blocks of the range (this wave streams every block of its slab)
  const long long i1 = min<long long>(hi, n1) - min<long long>(lo, n1);
  int left = static_cast<int>(i1 * nblk1 + (hi - lo - i1) * nblk0);
  Cur L;
  L.item = lo;
  settle(L);
  Cur Cc = L;
  static_for<0, R>([&](auto rc) {
    load(ring[decltype(rc)::value], L);
    advance(L);
  });
  auto kk_of = [&](const Cur& cu) __attribute__((always_inline)) {
    const int bip = cu.blk % cu.bpp;  // block within the phase
    return bip * (cu.fmt == kInt4 && WK == kInt4 ? 128 : 32);
  };
  while (left >= R) {
#pragma clang loop unroll(full)
    for (int r = 0; r < R; ++r) {
      if (Cc.blk % Cc.bpp == 0) begin_step(Cc);
      compute(ring[r], Cc, kk_of(Cc));
      load(ring[r], L);
      advance(L);
      advance(Cc);
    }
    left -= R;
  }
#pragma clang loop unroll(full)
  for (int r = 0; r < R; ++r) {
    if (r < left) {
      if (Cc.blk % Cc.bpp == 0) begin_step(Cc);
      compute(ring[r], Cc, kk_of(Cc));
      advance(Cc);
    }
  }
  item_end();
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

template <int WK, int G, int STAGE, int NC>
smoe_status launch_wide(const WArgs& a, long long items, hipStream_t st, const char* who) {
  auto kern = wide_ffn_kernel<WK, G, STAGE, NC>;
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

size_t wide_h_bytes(long long T, long long k, long long I, long long Is) {
  const long long bytes = 2 * (T * k * I + T * Is);
  return static_cast<size_t>((bytes + 255) / 256 * 256);
}

bool wide_applicable(const WideCall& c) {
  const long long S = static_cast<long long>(c.T) * c.k;
  return S >= kWideMinSlots && S <= kWideMaxSlots && c.E <= kMaxE && c.H % 128 == 0 &&
         c.I % 128 == 0 && c.Is % 128 == 0;
}

smoe_status wide_ffn(const WideCall& c, hipStream_t st, const char* who) {
  const long long S = static_cast<long long>(c.T) * c.k;
  const bool shared = c.Is > 0;
  // routed experts: chunks of 64 positions (4 MFMA column groups); the FP16
  // shared expert, which carries every token, in launches of its own with
  // chunks of 128 tokens (8 column groups), so that its weights stream half
  // as often. Two phase buffers of a chunk's rows fit the LDS either way.
  constexpr int kRoutedNC = 4, kSharedNC = 8;
  auto base = [&](WArgs& a, int nc) {
    a = WArgs{};
    a.sorted_slots = c.sorted_slots;
    a.offsets = c.offsets;
    a.slot_out = c.slot_out;
    a.k = c.k;
    a.S = static_cast<int>(S);
    a.T = c.T;
    a.H = c.H;
    a.n_groups = 1;
    a.kph = nc <= 4 ? 512 : 256;
    a.rstride = 2 * a.kph + kWPad;
    a.buf_bytes = 16 * nc * a.rstride;
  };
  _Float16* h_r = static_cast<_Float16*>(c.h);
  _Float16* h_s = h_r + S * c.I;
  auto fill = [&](WGroup& g, const void* w0, const void* w1, const void* s0, const void* s1,
                  int fmt, int N, int K, int ch, int kph, const void* src, void* out, int rows) {
    g.w[0] = static_cast<const uint8_t*>(w0);
    g.w[1] = static_cast<const uint8_t*>(w1 ? w1 : w0);
    g.s[0] = static_cast<const uint16_t*>(s0);
    g.s[1] = static_cast<const uint16_t*>(s1 ? s1 : s0);
    g.fmt = fmt;
    g.nblk = fmt == kInt4 ? K / 128 : K / 32;
    g.bpp = fmt == kInt4 ? kph / 128 : kph / 32;
    g.slabs = N / 16;
    g.tiles = (g.slabs + kWW - 1) / kWW;
    g.K = K;
    g.ch = ch;
    g.w_estride = static_cast<long long>(N) * g.nblk * kBlockBytes;
    g.s_estride = fmt == kInt4 ? static_cast<long long>(N) * (K / c.G) : 0;
    g.a = static_cast<const uint16_t*>(src);
    g.out = out;
    g.rows = rows;
  };
  // routed: group 0 of launches r1 / r2 (E experts)
  WArgs r1, r2;
  base(r1, kRoutedNC);
  base(r2, kRoutedNC);
  r1.E = r2.E = c.E;
  r2.zero_dropped = 1;
  const int chr = 16 * kRoutedNC;
  fill(r1.g[0], c.wg, c.wu, c.sg, c.su, c.fmt, c.I, c.H, chr, r1.kph, c.x, h_r,
       static_cast<int>(S));
  fill(r2.g[0], c.wd, nullptr, c.sd, nullptr, c.fmt, c.H, c.I, chr, r2.kph, h_r, c.slot_out,
       static_cast<int>(S));
  r1.g[1] = r1.g[0];
  r2.g[1] = r2.g[0];
  // shared: group 1 of launches s1 / s2, with no routed expert (E = 0)
  WArgs s1, s2;
  if (shared) {
    base(s1, kSharedNC);
    base(s2, kSharedNC);
    s1.E = s2.E = 0;
    s1.n_groups = s2.n_groups = 2;
    const int chs = 16 * kSharedNC;
    fill(s1.g[1], c.swg, c.swu, nullptr, nullptr, kFp16, c.Is, c.H, chs, s1.kph, c.x, h_s, c.T);
    fill(s2.g[1], c.swd, nullptr, nullptr, nullptr, kFp16, c.H, c.Is, chs, s2.kph, h_s,
         c.shared_out, c.T);
    s1.g[0] = s1.g[1];
    s2.g[0] = s2.g[1];
    s1.g[0].ch = s2.g[0].ch = chs;  // (no routed chunks: E = 0)
  }
  // upper bounds of the item counts (routed chunks <= min(E, S) + S / chunk)
  const long long items_r1 = (std::min<long long>(c.E, S) + S / chr) * r1.g[0].tiles;
  const long long items_r2 = (std::min<long long>(c.E, S) + S / chr) * r2.g[0].tiles;
  const long long items_s1 = shared ? (c.T + 16 * kSharedNC - 1) / (16 * kSharedNC) *
                                          static_cast<long long>(s1.g[1].tiles) : 0;
  const long long items_s2 = shared ? (c.T + 16 * kSharedNC - 1) / (16 * kSharedNC) *
                                          static_cast<long long>(s2.g[1].tiles) : 0;
  auto routed = [&](int stage) -> smoe_status {
    const WArgs& a = stage == 1 ? r1 : r2;
    const long long n = stage == 1 ? items_r1 : items_r2;
    if (c.fmt == kFp16)
      return stage == 1 ? launch_wide<kFp16, 128, 1, kRoutedNC>(a, n, st, who)
                        : launch_wide<kFp16, 128, 2, kRoutedNC>(a, n, st, who);
    switch (c.G) {
      case 32: return stage == 1 ? launch_wide<kInt4, 32, 1, kRoutedNC>(a, n, st, who)
                                 : launch_wide<kInt4, 32, 2, kRoutedNC>(a, n, st, who);
      case 64: return stage == 1 ? launch_wide<kInt4, 64, 1, kRoutedNC>(a, n, st, who)
                                 : launch_wide<kInt4, 64, 2, kRoutedNC>(a, n, st, who);
      default: return stage == 1 ? launch_wide<kInt4, 128, 1, kRoutedNC>(a, n, st, who)
                                 : launch_wide<kInt4, 128, 2, kRoutedNC>(a, n, st, who);
    }
  };
  smoe_status r = routed(1);
  if (r == SMOE_OK && shared) r = launch_wide<kFp16, 128, 1, kSharedNC>(s1, items_s1, st, who);
  if (r == SMOE_OK) r = routed(2);
  if (r == SMOE_OK && shared) r = launch_wide<kFp16, 128, 2, kSharedNC>(s2, items_s2, st, who);
  return r;
}

}  // namespace smoe
