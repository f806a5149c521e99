// smoe_w4a16_expert_ffn / smoe_fp16_expert_ffn: the fused multi-expert FFN.
//
// Specter paper: fused multi-expert draft kernel paragraph (the routed
// tokens are gathered by expert and all active experts' sub-computations run
// in one launch) and expert-wise verification paragraphs (tokens of each
// expert packed into one sub-batch, outputs scattered back). Design notes,
// "Streamlined Execution Engine": W4A16 dequantises INT4 weight tiles while
// computing with FP16 activations; FP32 reductions.
//
// Two launches per call, each over all active experts at once:
//   stage 1  g[p] = x_t . Wg^T,  u[p] = x_t . Wu^T          (fp32, p = sorted slot position)
//   stage 2  slot_out[s] = fp16(SiLU(g[p]) * u[p]) . Wd^T    (s = sorted_slots[p])
// SiLU(g) * u is formed (and rounded to fp16) while stage 2 stages its rows.
//
// The layer is bound by streaming the weights from HBM (a few slots per
// expert), so every weight byte is read once per slot chunk and the work is
// cut into many equal pieces spread evenly over the whole GPU:
//
// * Work list. The slots of each expert are cut into chunks of `csz` slots
//   (one chunk per expert when every token picks an expert at most once). A
//   row tile is 128 rows of gate and up (stage 1) or 256 rows of down
//   (stage 2): 16 / 32 rows per wave of an 8-wave workgroup. The reduction
//   dim K is cut into P parts of D blocks of 128 k. An item is (chunk, row
//   tile, part): every item streams the same number of weight bytes. Items
//   are numbered part-fastest; the persistent grid gives every busy
//   workgroup the same count q = ceil(n / nwg) of consecutive items. The
//   list is built on the device from expert_offsets (nothing is read back).
// * Split K. A workgroup adds the consecutive parts of a tile in registers.
//   A tile it holds whole is stored; a tile shared with a neighbouring
//   workgroup is added into the output with device-scope float atomics
//   (no return value, so nobody waits). Outputs that take atomics start at
//   zero: stage 1 clears slot_out for stage 2, and the g/u buffer of the
//   next call. The workspace keeps two g/u buffers and a two-word call
//   counter that picks the current one: stage 1 reads word 0 and writes
//   word 1, stage 2 reads word 1 and writes word 0, so no word is written
//   while another workgroup of the same launch may still read it.
// * Activations in LDS. The sorted slots and expert offsets come in with the
//   first round trip. A chunk's activation rows (x rows of its tokens in
//   stage 1, SiLU(g) * u of its positions in stage 2) are staged into LDS
//   when the chunk changes, k-permuted for INT4 (below) and padded by 16
//   bytes per row so the MFMA operand reads are bank-conflict free. The
//   first staging issues its loads before the weight prologue, so it never
//   waits behind it. Rows of K above the LDS budget are staged in phases.
// * Weight ring. Each wave streams its rows through a register ring of D
//   blocks that runs on across items; weights are the only global loads in
//   it, so the in-order vector memory counter never waits on anything but
//   the oldest block. One 16-byte load per lane covers 16 rows x 64
//   contiguous bytes per wave instruction. The INT4 group scales of an item
//   take one load per matrix: lane group g fetches block g's scale and each
//   block reads it from lane (d % 4, row) with a cross-lane shuffle.
//
// MFMA mapping (v_mfma_f32_16x16x32_f16, wave64): A = activations (16 slot
// rows x 32 k) from LDS, B = weights (32 k x 16 weight rows), D[slot][row].
// Lane l feeds slot / weight row l % 16 and k-slice l / 16, and holds D for
// slots 4*(l/16) + 0..3 of weight row l % 16 -- so every accumulator of a
// lane belongs to one weight row, and the INT4 group scale of that row is
// applied once per group in FP32 after the group's MFMAs. Chunks of more
// than 16 slots use a second 16-slot column group.
//
// INT4 dequantisation without lookup tables: a packed word w holds 8 codes;
// (w >> 4i) & 0x000F000F | 0x64006400 read as two fp16 values is
// (1024 + c_i, 1024 + c_{i+4}); subtracting 1032 gives c - 8 exactly. The
// eight values come out in k order 0,4,1,5,2,6,3,7, and the activations are
// staged with the same permutation within each group of 8.
//
// Word layout per 128-k block so that each MFMA's 32 k lie in one
// quantisation group (lane group g, MFMA step q):
//   G = 128: word 4g + q  (one 16-byte load of words 4g .. 4g+3);
//   G =  64: word 8(q/2) + 2g + q%2 (two 8-byte loads);
//   G =  32: word 4q + g  (four 4-byte loads).
// FP16 weights: step q, lane group g takes k = 32q + 8g .. +7 (four 16-byte
// loads per block; each wave instruction reads 16 rows x 64 bytes).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "smoe_internal.hpp"

namespace smoe {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { kInt4 = 0, kFp16 = 1 };
constexpr int kKB = 128;                   // k per block
constexpr int kWavesPerWg = 8;             // 4 waves per SIMD at two workgroups per CU
constexpr int kThreads = kWavesPerWg * kWave;
constexpr int kMaxChunk = 32;              // slots per chunk (two MFMA column groups)
constexpr int kTabInts = 2 * (kMaxE + 1);
constexpr int kTabBytes = (kTabInts * 4 + 15) / 16 * 16;  // offsets, chunk prefix
static_assert(kTabBytes % 16 == 0, "staged rows must start 16-byte aligned");
constexpr int kMaxSlotsLds = 1024;         // sorted slots kept whole in LDS up to this many
constexpr int kLdsPerCu = 160 * 1024;      // gfx950
constexpr int kLdsBudget = kLdsPerCu / 2;  // per workgroup: two workgroups per CU
constexpr int kRowPad = 16;                // bytes of padding per staged row
#ifndef SMOE_FFN_MAX_WG
#define SMOE_FFN_MAX_WG 512
#endif
#ifndef SMOE_FFN_D_INT4
#define SMOE_FFN_D_INT4 4
#endif
#ifndef SMOE_FFN_D_FP16
#define SMOE_FFN_D_FP16 1
#endif
constexpr int kMaxWg = SMOE_FFN_MAX_WG;    // persistent grid cap
constexpr int kDInt4 = SMOE_FFN_D_INT4;    // blocks per item, INT4 weights (2 KB per block and wave)
constexpr int kDFp16 = SMOE_FFN_D_FP16;    // blocks per item, FP16 weights (8 KB per block and wave)

struct FfnArgs {
  const uint16_t* x;            // stage 1 activations [T][K] (fp16 bits)
  const int32_t* sorted_slots;  // [S]
  const int32_t* offsets;       // [E+1]
  const uint8_t* w0;            // stage 1: gate; stage 2: down
  const uint8_t* w1;            // stage 1: up
  const uint16_t* s0;           // INT4 scales of w0 / w1 (fp16 bits)
  const uint16_t* s1;
  float* gu;                    // two g/u buffers, each [2][S][I] fp32
  float* out;                   // slot_out [S][H]: stage 1 clears it, stage 2 fills it
  int* epoch;                   // [2] call counter words
  long long gu_buf;             // floats per g/u buffer (2 * S * I)
  long long w_estride;          // bytes per expert
  long long s_estride;          // scale elements per expert
  int w_rstride;                // bytes per weight row
  int s_rstride;                // scale elements per row
  int E, k, S, K, N, I, H;
  int tiles;                    // row tiles per chunk
  int parts;                    // K parts per tile
  int csz;                      // slots per chunk = activation rows staged
  int chunks_upper;             // chunks the work list can hold
  int kp;                       // k-blocks per staged phase (a multiple of D)
  int stride;                   // LDS bytes per staged row
  int slots_lds;                // all S sorted slots copied to LDS at start
  int xs_off;                   // LDS byte offset of the staged rows
};

template <typename T, typename U>
__device__ __forceinline__ T bitcast(U u) {
  static_assert(sizeof(T) == sizeof(U), "size");
  T t;
  __builtin_memcpy(&t, &u, sizeof(T));
  return t;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Eight INT4 codes of one word -> (c - 8) as fp16, in k order 0,4,1,5,2,6,3,7.
// lo = 0x000F000F and magic = 0x64006400 are passed in registers so that
// each (w >> 4i) & lo | magic is a single v_and_or_b32.
__device__ __forceinline__ f16x8 dequant_word(uint32_t w, uint32_t lo, uint32_t magic) {
  const f16x2 bias = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
  const f16x2 v0 = bitcast<f16x2>((w & lo) | magic) - bias;
  const f16x2 v1 = bitcast<f16x2>(((w >> 4) & lo) | magic) - bias;
  const f16x2 v2 = bitcast<f16x2>(((w >> 8) & lo) | magic) - bias;
  const f16x2 v3 = bitcast<f16x2>(((w >> 12) & lo) | magic) - bias;
  f16x8 r;
  r[0] = v0[0]; r[1] = v0[1]; r[2] = v1[0]; r[3] = v1[1];
  r[4] = v2[0]; r[5] = v2[1]; r[6] = v3[0]; r[7] = v3[1];
  return r;
}

// Natural k order 0..7 -> 0,4,1,5,2,6,3,7 (matches dequant_word).
__device__ __forceinline__ u32x4 permute_k8(u32x4 d) {
  u32x4 e;
  e[0] = (d[0] & 0xFFFFu) | (d[2] << 16);
  e[1] = (d[0] >> 16) | (d[2] & 0xFFFF0000u);
  e[2] = (d[1] & 0xFFFFu) | (d[3] << 16);
  e[3] = (d[1] >> 16) | (d[3] & 0xFFFF0000u);
  return e;
}

// Word index (within a 128-k block) that MFMA step q of lane group g uses.
template <int G>
__device__ __forceinline__ int int4_word(int g, int q) {
  constexpr int per = G / 32;  // MFMA steps per quantisation group
  return (q / per) * (G / 8) + g * per + (q % per);
}

// k offset (within a 128-k block) of the 8 activations that lane group g
// feeds to MFMA step q.
template <int WK, int G>
__device__ __forceinline__ int a_koff(int g, int q) {
  return WK == kInt4 ? 8 * int4_word<G>(g, q) : 32 * q + 8 * g;
}

template <int WK, int G>
struct Block {
  static constexpr int NW = WK == kInt4 ? 1 : 4;   // u32x4 per matrix
  static constexpr int NQ = WK == kInt4 ? kKB / G : 1;
  u32x4 w[2][NW];
};

// One item: part `part` of row tile `tile` of chunk `chunk` (expert e,
// sorted positions [seg0, seg0 + m)).
struct Item {
  int chunk, tile, part, e, seg0, m;
};

__device__ __forceinline__ Item decode_item(const int* s_off, const int* s_cp, int E, int tiles,
                                            int parts, int csz, int item) {
  Item it;
  const int ct = item / parts;
  it.part = item - ct * parts;
  it.chunk = ct / tiles;
  it.tile = ct - it.chunk * tiles;
  const int lane = lane_id();
  int found = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    if (e < E && s_cp[e] <= it.chunk && it.chunk < s_cp[e + 1]) found = e;
  }
  const uint64_t mask = __ballot(found >= 0);
  const int src = mask ? __ffsll(static_cast<long long>(mask)) - 1 : 0;
  it.e = uniform(__shfl(found, src, kWave));
  it.seg0 = s_off[it.e] + (it.chunk - s_cp[it.e]) * csz;
  it.m = min(csz, s_off[it.e + 1] - it.seg0);
  return it;
}

template <int WK, int G, int STAGE, int NC, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void ffn_kernel(
    FfnArgs a) {
  using Blk = Block<WK, G>;
  constexpr int NQ = Blk::NQ;
  extern __shared__ __align__(16) uint8_t smem[];
  int* s_off = reinterpret_cast<int*>(smem);
  int* s_cp = s_off + (kMaxE + 1);
  int* s_slots = reinterpret_cast<int*>(smem + kTabBytes);  // all slots, or the chunk's
  uint8_t* xs = smem + a.xs_off;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int E = a.E;
  const int P = a.parts;
  const int nblk = a.K / kKB;
  const int b = blockIdx.x;

  // ---- one round trip for the work list: expert offsets, sorted slots
  // (when they fit LDS) and the call counter
  static_assert(kThreads > kMaxE, "one offset per thread");
  const int offv = tid <= E ? a.offsets[tid] : 0;
  constexpr int kSlotsPer = kMaxSlotsLds / kThreads;
  int slv[kSlotsPer];
  if (a.slots_lds) {
#pragma unroll
    for (int j = 0; j < kSlotsPer; ++j) {
      const int i = tid + j * kThreads;
      slv[j] = i < a.S ? a.sorted_slots[i] : -1;
    }
  }
  const int ep = a.epoch[STAGE == 1 ? 0 : 1];
  // the g/u buffer of this call
  float* gu = a.gu + ((STAGE == 1 ? ep : ep - 1) & 1) * a.gu_buf;
  if (tid <= E) s_off[tid] = min(max(offv, 0), a.S);  // clamped to [0, S]
  if (a.slots_lds) {
#pragma unroll
    for (int j = 0; j < kSlotsPer; ++j)
      if (tid + j * kThreads < a.S) s_slots[tid + j * kThreads] = slv[j];
  }
  if (b == 0 && tid == 0) a.epoch[STAGE == 1 ? 1 : 0] = ep + 1 - (STAGE == 1 ? 0 : 1);
  __syncthreads();

  // ---- work list: chunk prefix over experts
  if (wave == 0) {
    int n[4], tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      n[i] = e < E ? (max(s_off[e + 1] - s_off[e], 0) + a.csz - 1) / a.csz : 0;
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
  __syncthreads();
  // (inconsistent offsets could describe more chunks than the list holds;
  // the excess is ignored)
  const int n_items = min(s_cp[E], a.chunks_upper) * a.tiles * P;
  // q items per workgroup and only ceil(n_items / q) workgroups busy, so
  // every busy workgroup streams the same number of bytes
  const int q = (n_items + gridDim.x - 1) / gridDim.x;
  const int i0 = b * q;
  const int i1 = min(n_items, i0 + q);

  // Stage 1 clears what split tiles will add into: slot_out (for stage 2)
  // and the other g/u buffer (for the next call). Each workgroup clears its
  // share once its own items are done (or at once if it has none).
  auto clear_share = [&]() {
    if (STAGE != 1) return;
    float* other = a.gu + ((ep + 1) & 1) * a.gu_buf;
    const long long n_gu = a.gu_buf / 4, n_out = static_cast<long long>(a.S) * a.H / 4;
    const long long tot = n_gu + n_out;
    const long long per = (tot + gridDim.x - 1) / gridDim.x;
    const long long lo = per * b, hi = min(tot, lo + per);
    for (long long i = lo + tid; i < hi; i += kThreads) {
      f32x4* dst = i < n_gu ? reinterpret_cast<f32x4*>(other) + i
                            : reinterpret_cast<f32x4*>(a.out) + (i - n_gu);
      *dst = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  if (i0 >= i1) {  // whole workgroup
    clear_share();
    return;
  }

  // weight row of matrix m for this lane in row tile `tile`
  auto row_of = [&](int tile, int m) {
    return STAGE == 1 ? tile * (kWavesPerWg * 16) + wave * 16 + r16
                      : tile * (kWavesPerWg * 32) + wave * 32 + m * 16 + r16;
  };
  const int lane_kb = WK == kInt4 ? (G == 128 ? 16 * g : (G == 64 ? 8 * g : 4 * g)) : 16 * g;

  // ---- load cursor
  const uint8_t* wp[2];
  const uint16_t* sp[2];
  int l_blk0 = 0;  // first block of the item being loaded
  auto set_load_item = [&](int item) {
    const Item it = decode_item(s_off, s_cp, E, a.tiles, P, a.csz, item);
    l_blk0 = it.part * D;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int row = min(row_of(it.tile, m), a.N - 1);  // rows past N: loaded, never stored
      const uint8_t* wm = (STAGE == 1 && m == 1) ? a.w1 : a.w0;
      wp[m] = wm + it.e * a.w_estride + static_cast<long long>(row) * a.w_rstride + lane_kb;
      if (WK == kInt4) {
        const uint16_t* sm = (STAGE == 1 && m == 1) ? a.s1 : a.s0;
        sp[m] = sm + it.e * a.s_estride + static_cast<long long>(row) * a.s_rstride;
      }
    }
  };
  auto load = [&](Blk& r, int blk) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (WK == kInt4) {
        const uint8_t* base = wp[m] + blk * (kKB / 2);
        if (G == 128) {
          r.w[m][0] = *reinterpret_cast<const u32x4*>(base);
        } else if (G == 64) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(base);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(base + 32);
          r.w[m][0] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            r.w[m][0][qq] = *reinterpret_cast<const uint32_t*>(base + 16 * qq);
        }
      } else {
        const uint8_t* base = wp[m] + blk * (kKB * 2);
#pragma unroll
        for (int c = 0; c < 4; ++c) r.w[m][c] = *reinterpret_cast<const u32x4*>(base + 64 * c);
      }
    }
  };

  // INT4 group scales of an item, one load per matrix: lane group g holds
  // the scales of blocks blk0 + g + 4j of its row (NS words each); block d
  // reads them from lane (d % 4, row) with a cross-lane shuffle.
  static_assert(WK != kInt4 || D % 4 == 0, "INT4 items are whole groups of 4 blocks");
  constexpr int DJ = (D + 3) / 4;
  constexpr int NS = NQ == 4 ? 2 : 1;
  uint32_t sring[2][DJ][NS], scur[2][DJ][NS];
  auto load_scales = [&](int blk0) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
        const uint16_t* sptr = sp[m] + min(blk0 + g + 4 * j, nblk - 1) * NQ;
        if (NQ == 1) {
          sring[m][j][0] = *sptr;
        } else if (NQ == 2) {
          sring[m][j][0] = *reinterpret_cast<const uint32_t*>(sptr);
        } else {
          const u32x2 v = *reinterpret_cast<const u32x2*>(sptr);
          sring[m][j][0] = v[0];
          sring[m][j][1] = v[1];
        }
      }
  };

  f32x4 acc[2][NC];
  uint32_t dq_lo = 0x000F000Fu, dq_magic = 0x64006400u;
  asm volatile("" : "+v"(dq_lo), "+v"(dq_magic));  // keep the masks in VGPRs

  // Slot r of chunk `it` (from the full copy in LDS, or the chunk's copy).
  auto chunk_slot = [&](const Item& it, int r) {
    return a.slots_lds ? s_slots[it.seg0 + r] : s_slots[r];
  };
  // A operand rows (LDS byte offsets) of this lane; lanes past the chunk's
  // slots read a staged row and their results are dropped.
  int arow[NC];
#pragma unroll
  for (int cg = 0; cg < NC; ++cg) arow[cg] = min(16 * cg + r16, a.csz - 1) * a.stride;

  auto compute = [&](const Blk& r, int bp, int d, auto nce_tag) {
    constexpr int NCE = decltype(nce_tag)::value;
    f16x8 A[NCE][4];
#pragma unroll
    for (int cg = 0; cg < NCE; ++cg) {
      const uint8_t* ar = xs + arow[cg] + bp * (kKB * 2);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        A[cg][qq] = *reinterpret_cast<const f16x8*>(ar + 2 * a_koff<WK, G>(g, qq));
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (WK == kInt4) {
        f16x8 B[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) B[qq] = dequant_word(r.w[m][0][qq], dq_lo, dq_magic);
        constexpr int per = G / 32;
#pragma unroll
        for (int grp = 0; grp < NQ; ++grp) {
          const int src = (d & 3) * 16 + r16;
          const uint32_t word = __shfl(scur[m][d >> 2][NQ == 4 ? (grp >> 1) : 0], src, kWave);
          const uint32_t sbits = (NQ == 4) ? (word >> (16 * (grp & 1))) : (word >> (16 * grp));
          const float sc =
              static_cast<float>(bitcast<_Float16>(static_cast<uint16_t>(sbits & 0xFFFFu)));
#pragma unroll
          for (int cg = 0; cg < NCE; ++cg) {
            f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int qq = 0; qq < per; ++qq)
              t = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[cg][grp * per + qq],
                                                         B[grp * per + qq], t, 0, 0, 0);
            acc[m][cg] += sc * t;
          }
        }
      } else {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const f16x8 Bq = bitcast<f16x8>(r.w[m][qq]);
#pragma unroll
          for (int cg = 0; cg < NCE; ++cg)
            acc[m][cg] =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(A[cg][qq], Bq, acc[m][cg], 0, 0, 0);
        }
      }
    }
  };

  // Staged activations, eight columns at a time: stage 1 copies x of the
  // slot's token; stage 2 forms fp16(SiLU(g) * u) of the position. The loads
  // (load_raw) and the conversion (finish) are split so that a batch of
  // loads is in flight before anything waits on it.
  struct Raw1 {
    u32x4 v;
  };
  struct Raw2 {
    f32x4 g0, g1, u0, u1;
  };
  using Raw = typename std::conditional<STAGE == 1, Raw1, Raw2>::type;
  // Returns false for a row that is not staged (a dropped slot); its loads
  // stay in bounds.
  auto load_raw = [&](const Item& it, int r, int col, Raw& raw) -> bool {
    if constexpr (STAGE == 1) {
      const int slot = chunk_slot(it, r);
      const bool ok = slot >= 0 && slot < a.S;
      raw.v = *reinterpret_cast<const u32x4*>(
          a.x + static_cast<long long>(ok ? slot / a.k : 0) * a.K + col);
      return ok;
    } else {
      const float* gr = gu + static_cast<long long>(it.seg0 + r) * a.I + col;
      const float* ur = gr + static_cast<long long>(a.S) * a.I;
      raw.g0 = *reinterpret_cast<const f32x4*>(gr);
      raw.g1 = *reinterpret_cast<const f32x4*>(gr + 4);
      raw.u0 = *reinterpret_cast<const f32x4*>(ur);
      raw.u1 = *reinterpret_cast<const f32x4*>(ur + 4);
      return true;
    }
  };
  auto finish = [&](const Raw& raw) -> u32x4 {
    if constexpr (STAGE == 1) {
      return WK == kInt4 ? permute_k8(raw.v) : raw.v;
    } else {
      f16x8 h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = static_cast<_Float16>(raw.g0[i] / (1.0f + __expf(-raw.g0[i])) * raw.u0[i]);
        h[4 + i] = static_cast<_Float16>(raw.g1[i] / (1.0f + __expf(-raw.g1[i])) * raw.u1[i]);
      }
      const u32x4 v = bitcast<u32x4>(h);
      return WK == kInt4 ? permute_k8(v) : v;
    }
  };

  // Stage the activation rows of chunk `it`, k-blocks [phase*kp, ...), into
  // LDS. `mid` runs right after the first batch of loads is issued, so the
  // weight prologue can go out behind it without the staging waiting on it.
  auto stage_rows = [&](const Item& it, int phase, auto batch_tag, auto&& mid) {
    constexpr int NB = decltype(batch_tag)::value;  // pieces in flight per thread
    __syncthreads();  // every wave is done with the previous rows
    if (!a.slots_lds) {
      if (tid < it.m) s_slots[tid] = a.sorted_slots[it.seg0 + tid];
      __syncthreads();
    }
    const int kb0 = phase * a.kp;
    const int npr = min(a.kp, nblk - kb0) * (kKB / 8);  // 16-byte pieces per row
    const int tot = it.m * npr;
    for (int base = 0; base < tot; base += NB * kThreads) {
      Raw raw[NB];
      int dst[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int i = min(base + j * kThreads + tid, tot - 1);
        const int r = i / npr, c = i - r * npr;
        const bool ok = load_raw(it, r, kb0 * kKB + 8 * c, raw[j]);
        dst[j] = (ok && base + j * kThreads + tid < tot) ? r * a.stride + 16 * c : -1;
      }
      if (base == 0) mid();
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (dst[j] >= 0) *reinterpret_cast<u32x4*>(xs + dst[j]) = finish(raw[j]);
    }
    __syncthreads();
  };

  // Write the sums of a tile; a tile split with other workgroups is added
  // into the (zeroed) output with device-scope atomics.
  auto write_tile = [&](const Item& it, bool whole) {
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * cg + 4 * g + i;
        if (rr >= it.m) continue;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int row = row_of(it.tile, STAGE == 1 ? 0 : m);
          if (row >= a.N) continue;
          float* dst;
          if (STAGE == 1) {
            dst = gu + static_cast<long long>(m) * a.S * a.I +
                  static_cast<long long>(it.seg0 + rr) * a.I + row;
          } else {
            const int slot = chunk_slot(it, rr);
            if (slot < 0 || slot >= a.S) continue;
            dst = a.out + static_cast<long long>(slot) * a.H + row;
          }
          if (whole)
            *dst = acc[m][cg][i];
          else
            __hip_atomic_fetch_add(dst, acc[m][cg][i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  };

  // ---- prologue: stage the first chunk, the first item's blocks in flight
  Item ci = decode_item(s_off, s_cp, E, a.tiles, P, a.csz, i0);
  set_load_item(i0);
  Blk ring[D];
  int staged_chunk = ci.chunk, staged_phase = (ci.part * D) / a.kp;
  stage_rows(ci, staged_phase, std::integral_constant<int, STAGE == 1 ? 4 : 2>(), [&]() {
    if (WK == kInt4) load_scales(l_blk0);
#pragma unroll
    for (int d = 0; d < D; ++d) load(ring[d], min(l_blk0 + d, nblk - 1));
  });
  int seg_pa = ci.part;  // first part of the tile accumulated so far

  for (int item = i0; item < i1; ++item) {
    const int blk0 = ci.part * D;
    if (item == i0 || ci.part == 0) {
      seg_pa = ci.part;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) acc[m][cg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int phase = blk0 / a.kp;
    if (ci.chunk != staged_chunk || phase != staged_phase) {
      stage_rows(ci, phase, std::integral_constant<int, STAGE == 1 ? 2 : 1>(), []() {});
      staged_chunk = ci.chunk;
      staged_phase = phase;
    }

    // the load cursor moves to the next item
    const bool l_live = item + 1 < i1;
    if (l_live) set_load_item(item + 1);

    const bool wide = NC == 2 && ci.m > 16;
    const int bp0 = blk0 - phase * a.kp;
    if (WK == kInt4) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < DJ; ++j)
#pragma unroll
          for (int t = 0; t < NS; ++t) scur[m][j][t] = sring[m][j][t];
      if (l_live) load_scales(l_blk0);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (blk0 + d < nblk) {
        if (wide)
          compute(ring[d], bp0 + d, d, std::integral_constant<int, NC>());
        else
          compute(ring[d], bp0 + d, d, std::integral_constant<int, 1>());
      }
      if (l_live) load(ring[d], min(l_blk0 + d, nblk - 1));
    }

    if (item + 1 == i1 || ci.part == P - 1) write_tile(ci, seg_pa == 0 && ci.part == P - 1);
    if (item + 1 < i1) ci = decode_item(s_off, s_cp, E, a.tiles, P, a.csz, item + 1);
  }
  clear_share();
}

// ------------------------------------------------------------------ host side

int cu_count() {
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

// Launch plan of one stage: K parts, LDS phase length kp (a multiple of D,
// so phases start on item boundaries), staged row stride, LDS layout.
struct StagePlan {
  int parts, kp, stride, lds, items, slots_lds, xs_off;
};

StagePlan plan_stage(int D, int csz, int S, int K, int chunks_upper, int tiles) {
  StagePlan p{};
  const int nblk = K / kKB;
  p.parts = (nblk + D - 1) / D;
  p.items = chunks_upper * tiles * p.parts;
  p.slots_lds = S <= kMaxSlotsLds ? 1 : 0;
  p.xs_off = kTabBytes + ((p.slots_lds ? S : kMaxChunk) * 4 + 15) / 16 * 16;
  const int per_row = (kLdsBudget - p.xs_off) / csz;
  const int kp_cap = std::max(1, (per_row - kRowPad) / (kKB * 2));
  const int kpmax = std::max(D, kp_cap / D * D);
  const int phases = (nblk + kpmax - 1) / kpmax;
  const int per_phase = (nblk + phases - 1) / phases;
  p.kp = (per_phase + D - 1) / D * D;
  p.stride = std::min(p.kp, nblk) * kKB * 2 + kRowPad;
  p.lds = p.xs_off + csz * p.stride;
  return p;
}

template <int WK, int G, int STAGE, int NC>
smoe_status launch_stage(const FfnArgs& a, const StagePlan& p, hipStream_t st) {
  constexpr int D = WK == kInt4 ? kDInt4 : kDFp16;
  auto kern = ffn_kernel<WK, G, STAGE, NC, D>;
  static std::atomic<int> attr_done{0};
  if (!attr_done.load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) != hipSuccess) {
      set_error("expert_ffn: cannot raise the dynamic LDS limit to %d bytes", kLdsBudget);
      return SMOE_EHIP;
    }
    attr_done.store(1, std::memory_order_release);
  }
  const int per_cu = 2 * p.lds <= kLdsPerCu ? 2 : 1;
  const int nwg = std::max(1, std::min({p.items, per_cu * cu_count(), kMaxWg}));
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(kThreads), p.lds, st, a);
  return check_launch(STAGE == 1 ? "expert_ffn stage 1" : "expert_ffn stage 2");
}

template <int WK, int G, int NC>
smoe_status launch_ffn(const FfnArgs& a1, const FfnArgs& a2, const StagePlan& p1,
                       const StagePlan& p2, hipStream_t st) {
  smoe_status s = launch_stage<WK, G, 1, NC>(a1, p1, st);
  if (s != SMOE_OK) return s;
  return launch_stage<WK, G, 2, NC>(a2, p2, st);
}

// Slots per chunk: two 16-slot MFMA column groups when one expert is
// expected to hold more than 16 of the window's slots (long windows, or few
// experts such as a shared expert that every token uses), else one (an
// expert with more slots then gets a second chunk and reads its weights
// twice, which at these windows is rare).
int chunk_slots(long long T, long long k, long long E) {
  const long long S = T * k;
  const bool wide = T > 16 && (T > 24 || S > 8 * std::min(E, S));
  return static_cast<int>(std::max(1ll, std::min(T, static_cast<long long>(wide ? kMaxChunk : 16))));
}

// Row tiles of a matrix with N output rows, rows_per_wave rows per wave.
int tiles_of(long long N, int rows_per_wave) {
  const long long rows = static_cast<long long>(kWavesPerWg) * rows_per_wave;
  return static_cast<int>((N + rows - 1) / rows);
}

// Workspace layout: call counter (2 words, padded to 256 bytes) | two g/u
// buffers of [2][S][I] fp32.
constexpr size_t kEpochBytes = 256;
size_t workspace_bytes(long long T, long long k, long long I) {
  return kEpochBytes + static_cast<size_t>(4 * T * k * I) * sizeof(float);
}

smoe_status check_common(const char* who, const void* x, int T, int k, int E, int H, int I,
                         const int32_t* sorted_slots, const int32_t* offsets,
                         const void* workspace, size_t ws_bytes, const float* slot_out) {
  SMOE_REQUIRE(T >= 0 && k > 0 && E > 0 && H > 0 && I > 0, SMOE_EINVAL,
               "%s: need T >= 0 and k, E, H, I > 0 (T=%d k=%d E=%d H=%d I=%d)", who, T, k, E, H, I);
  SMOE_REQUIRE(E <= kMaxE && k <= kMaxK && k <= E, SMOE_EUNSUPPORTED,
               "%s: need E <= 256 and k <= min(8, E) (E=%d k=%d)", who, E, k);
  SMOE_REQUIRE(H % 128 == 0 && I % 128 == 0, SMOE_EUNSUPPORTED,
               "%s: H and I must be multiples of 128 (H=%d I=%d)", who, H, I);
  SMOE_REQUIRE(H <= 16384 && I <= 32768, SMOE_EUNSUPPORTED,
               "%s: need H <= 16384 and I <= 32768 (H=%d I=%d)", who, H, I);
  SMOE_REQUIRE(static_cast<long long>(T) * k < (1ll << 24) &&
                   static_cast<long long>(T) * k * std::max(H, I) < (1ll << 31),
               SMOE_EUNSUPPORTED, "%s: T*k must be below 2^24 and T*k*max(H, I) below 2^31",
               who);
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(x && sorted_slots && offsets && workspace && slot_out, SMOE_EINVAL,
               "%s: null pointer", who);
  const size_t need = workspace_bytes(T, k, I);
  SMOE_REQUIRE(ws_bytes >= need, SMOE_EINVAL, "%s: workspace of %zu bytes is below the %zu needed",
               who, ws_bytes, need);
  SMOE_REQUIRE(aligned16(x) && (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0 &&
                   aligned16(slot_out),
               SMOE_EINVAL,
               "%s: x and slot_out must be 16-byte aligned, the workspace 256-byte aligned", who);
  return SMOE_OK;
}

// Fill the stage arguments and launch plans shared by both weight formats.
void fill_args(int D, FfnArgs& a1, FfnArgs& a2, StagePlan& p1, StagePlan& p2, int& nc,
               const void* x, int T, int k, int E, int H, int I, const int32_t* sorted_slots,
               const int32_t* offsets, void* workspace, float* slot_out) {
  const int S = T * k;
  const int csz = chunk_slots(T, k, E);
  nc = csz > 16 ? 2 : 1;
  const int chunks_upper = std::min(E, S) + S / csz;
  uint8_t* wsb = static_cast<uint8_t*>(workspace);
  a1 = FfnArgs{};
  a1.x = static_cast<const uint16_t*>(x);
  a1.sorted_slots = sorted_slots;
  a1.offsets = offsets;
  a1.epoch = reinterpret_cast<int*>(wsb);
  a1.gu = reinterpret_cast<float*>(wsb + kEpochBytes);
  a1.gu_buf = 2ll * S * I;
  a1.out = slot_out;
  a1.E = E; a1.k = k; a1.S = S; a1.I = I; a1.H = H;
  a1.K = H; a1.N = I;
  a1.tiles = tiles_of(I, 16);
  a1.csz = csz;
  a1.chunks_upper = chunks_upper;
  p1 = plan_stage(D, csz, S, H, chunks_upper, a1.tiles);
  a1.parts = p1.parts;
  a1.kp = p1.kp;
  a1.stride = p1.stride;
  a1.slots_lds = p1.slots_lds;
  a1.xs_off = p1.xs_off;

  a2 = a1;
  a2.K = I; a2.N = H;
  a2.tiles = tiles_of(H, 32);
  p2 = plan_stage(D, csz, S, I, chunks_upper, a2.tiles);
  a2.parts = p2.parts;
  a2.kp = p2.kp;
  a2.stride = p2.stride;
  a2.slots_lds = p2.slots_lds;
  a2.xs_off = p2.xs_off;
}

}  // namespace
}  // namespace smoe

using namespace smoe;

extern "C" size_t smoe_ffn_workspace_bytes(int T, int k, int E, int H, int I) {
  if (T <= 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0) return 0;
  return workspace_bytes(T, k, I);
}

extern "C" smoe_status smoe_w4a16_expert_ffn(const void* x, int T, int k, int E, int H, int I,
                                             int group_size, const uint32_t* wg_q,
                                             const void* wg_s, const uint32_t* wu_q,
                                             const void* wu_s, const uint32_t* wd_q,
                                             const void* wd_s, const int32_t* sorted_slots,
                                             const int32_t* expert_offsets, void* workspace,
                                             size_t workspace_bytes_, float* slot_out,
                                             void* stream) {
  clear_error();
  SMOE_REQUIRE(group_size == 32 || group_size == 64 || group_size == 128, SMOE_EUNSUPPORTED,
               "w4a16_expert_ffn: group size must be 32, 64 or 128 (got %d)", group_size);
  smoe_status st = check_common("w4a16_expert_ffn", x, T, k, E, H, I, sorted_slots,
                                expert_offsets, workspace, workspace_bytes_, slot_out);
  if (st != SMOE_OK) return st;
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(wg_q && wg_s && wu_q && wu_s && wd_q && wd_s, SMOE_EINVAL,
               "w4a16_expert_ffn: null weight pointer");
  SMOE_REQUIRE(aligned16(wg_q) && aligned16(wu_q) && aligned16(wd_q), SMOE_EINVAL,
               "w4a16_expert_ffn: packed weights must be 16-byte aligned");
  SMOE_REQUIRE(((reinterpret_cast<uintptr_t>(wg_s) | reinterpret_cast<uintptr_t>(wu_s) |
                 reinterpret_cast<uintptr_t>(wd_s)) & 7u) == 0,
               SMOE_EINVAL, "w4a16_expert_ffn: scales must be 8-byte aligned");

  FfnArgs a1, a2;
  StagePlan p1, p2;
  int nc;
  fill_args(kDInt4, a1, a2, p1, p2, nc, x, T, k, E, H, I, sorted_slots, expert_offsets,
            workspace, slot_out);
  a1.w0 = reinterpret_cast<const uint8_t*>(wg_q);
  a1.w1 = reinterpret_cast<const uint8_t*>(wu_q);
  a1.s0 = static_cast<const uint16_t*>(wg_s);
  a1.s1 = static_cast<const uint16_t*>(wu_s);
  a1.w_rstride = H / 2;
  a1.w_estride = static_cast<long long>(a1.w_rstride) * I;
  a1.s_rstride = H / group_size;
  a1.s_estride = static_cast<long long>(a1.s_rstride) * I;

  a2.w0 = reinterpret_cast<const uint8_t*>(wd_q);
  a2.w1 = nullptr;
  a2.s0 = static_cast<const uint16_t*>(wd_s);
  a2.s1 = nullptr;
  a2.w_rstride = I / 2;
  a2.w_estride = static_cast<long long>(a2.w_rstride) * H;
  a2.s_rstride = I / group_size;
  a2.s_estride = static_cast<long long>(a2.s_rstride) * H;

  hipStream_t s = as_stream(stream);
#define SMOE_FFN_NC(G)                                  \
  (nc == 2 ? launch_ffn<kInt4, G, 2>(a1, a2, p1, p2, s) \
           : launch_ffn<kInt4, G, 1>(a1, a2, p1, p2, s))
  switch (group_size) {
    case 32: return SMOE_FFN_NC(32);
    case 64: return SMOE_FFN_NC(64);
    default: return SMOE_FFN_NC(128);
  }
#undef SMOE_FFN_NC
}

extern "C" smoe_status smoe_fp16_expert_ffn(const void* x, int T, int k, int E, int H, int I,
                                            const void* wg, const void* wu, const void* wd,
                                            const int32_t* sorted_slots,
                                            const int32_t* expert_offsets, void* workspace,
                                            size_t workspace_bytes_, float* slot_out,
                                            void* stream) {
  clear_error();
  smoe_status st = check_common("fp16_expert_ffn", x, T, k, E, H, I, sorted_slots,
                                expert_offsets, workspace, workspace_bytes_, slot_out);
  if (st != SMOE_OK) return st;
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(wg && wu && wd, SMOE_EINVAL, "fp16_expert_ffn: null weight pointer");
  SMOE_REQUIRE(aligned16(wg) && aligned16(wu) && aligned16(wd), SMOE_EINVAL,
               "fp16_expert_ffn: weights must be 16-byte aligned");

  FfnArgs a1, a2;
  StagePlan p1, p2;
  int nc;
  fill_args(kDFp16, a1, a2, p1, p2, nc, x, T, k, E, H, I, sorted_slots, expert_offsets,
            workspace, slot_out);
  a1.w0 = static_cast<const uint8_t*>(wg);
  a1.w1 = static_cast<const uint8_t*>(wu);
  a1.w_rstride = H * 2;
  a1.w_estride = static_cast<long long>(a1.w_rstride) * I;
  a2.w0 = static_cast<const uint8_t*>(wd);
  a2.w1 = nullptr;
  a2.w_rstride = I * 2;
  a2.w_estride = static_cast<long long>(a2.w_rstride) * H;
  hipStream_t s = as_stream(stream);
  return nc == 2 ? launch_ffn<kFp16, 128, 2>(a1, a2, p1, p2, s)
                 : launch_ffn<kFp16, 128, 1>(a1, a2, p1, p2, s);
}
