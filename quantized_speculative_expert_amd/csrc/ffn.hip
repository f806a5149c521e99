// smoe_w4a16_expert_ffn / smoe_fp16_expert_ffn: the fused multi-expert FFN.
//
// Specter paper: fused multi-expert draft kernel paragraph (the routed
// tokens are gathered by expert and all active experts' sub-computations run
// in one launch), expert-wise verification paragraphs (tokens of each expert
// packed into one sub-batch, outputs scattered back) and the hybrid-precision
// layout (always-on shared experts stay FP16). Design notes, "Streamlined
// Execution Engine": W4A16 dequantises INT4 weight tiles while computing
// with FP16 activations; FP32 reductions.
//
// Two launches per call, each over all active routed experts and the
// optional FP16 shared expert at once:
//   stage 1  g[p] = x_t . Wg^T,  u[p] = x_t . Wu^T          (fp32, p = sorted slot position)
//   stage 2  out[s] = fp16(SiLU(g[p]) * u[p]) . Wd^T          (s = sorted_slots[p])
// SiLU(g) * u is formed (and rounded to fp16) while stage 2 stages its rows.
// The shared expert takes every token in order (its slot t is token t).
//
// The layer is bound by streaming the weights from HBM (a few slots per
// expert), so every weight byte is read once per slot chunk and the work is
// cut into many equal pieces spread evenly over the whole GPU:
//
// * Blocks. A block is 64 bytes of one weight row: 128 k of INT4 codes or
//   32 k of FP16 values, so both formats fill the same register ring and an
//   item (D blocks) streams the same bytes whatever the format.
// * Work list. The slots of each expert are cut into chunks of `csz` slots
//   (one chunk per expert when every token picks an expert at most once). A
//   row tile is 128 rows of gate and up (stage 1) or 256 rows of down
//   (stage 2): 16 / 32 rows per wave of an 8-wave workgroup. The reduction
//   dim K is cut into parts of D blocks (4 in stage 1, 3 in stage 2, whose
//   work is smaller and so is cut finer; 2 in an INT4 stage 1 with 32-slot
//   chunks and x not resident, whose accumulators and staged rows leave no
//   registers for a deeper ring without spilling). An item is (chunk, row tile, part);
//   the shared expert's items come first, the routed experts' after them,
//   so the static runs below hold the shared tiles (every token: the
//   widest items) and the dynamic tail is made of routed items.
//   The list is built on the device from expert_offsets (nothing is read
//   back). Each workgroup of the persistent grid first takes a run of
//   consecutive items (nine tenths of an even share); the rest goes out
//   in units of two consecutive items through a few device-scope ticket
//   counters, so workgroups that stream faster take more of it and the
//   grid finishes together instead of waiting on its slowest members.
// * Split K. A workgroup adds the consecutive parts of a tile in registers.
//   A tile it holds whole is stored; a tile shared with other workgroups is
//   added into the output with device-scope float atomics (no return value,
//   so nobody waits). Outputs that take atomics start at zero: stage 1
//   clears slot_out and shared_out for stage 2, and the g/u buffer of the
//   next call. The workspace keeps two g/u buffers and a two-word call
//   counter that picks the current one: stage 1 reads word 0 and writes
//   word 1, stage 2 reads word 1 and writes word 0, so no word is written
//   while another workgroup of the same launch may still read it. Each
//   stage likewise resets the other stage's ticket counters for its next
//   launch.
// * Activations in LDS. The sorted slots and expert offsets come in with the
//   first round trip. A chunk's activation rows (x rows of its tokens in
//   stage 1, SiLU(g) * u of its positions in stage 2) are staged into LDS
//   when the chunk changes, k-permuted for INT4 (below) and padded by 16
//   bytes per row so the MFMA operand reads are bank-conflict free. The
//   first staging issues its loads before the weight prologue, so it never
//   waits behind it. Rows longer than the LDS budget are staged in phases.
//   When all T rows of x fit (short windows), stage 1 instead stages x
//   whole once per launch and an item's A rows are the tokens of its
//   slots: no item restages, and the FP16 shared weights take the INT4
//   k-permutation in registers.
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
// (1024 + c_i, 1024 + c_{i+4}); subtracting 1032 gives c - 8 exactly (the
// odd i are read in place, see dequant_word). The eight values come out in
// k order 0,4,1,5,2,6,3,7, and the activations are staged with the same
// permutation within each group of 8.
//
// INT4 word layout per block so that each MFMA's 32 k lie in one
// quantisation group (lane group g, MFMA step q):
//   G = 128: word 4g + q  (one 16-byte load of words 4g .. 4g+3);
//   G =  64: word 8(q/2) + 2g + q%2 (two 8-byte loads);
//   G =  32: word 4q + g  (four 4-byte loads).
// In the tiled layout (smoe_tile_weights) each lane's four words already
// sit in step order in 16 consecutive bytes, one load for every G.
// FP16 block: one MFMA step, lane group g takes k = 8g .. 8g+7 of the block.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "ffn_device.hpp"
#include "decode.hpp"
#include "ffn_wide.hpp"
#include "smoe_blocks.hpp"  // route_check (the layer call validates every step)

namespace smoe {
namespace {

constexpr int kWavesPerWg = 8;             // 4 waves per SIMD at two workgroups per CU
constexpr int kThreads = kWavesPerWg * kWave;
constexpr int kMaxChunk = 32;              // slots per chunk (two MFMA column groups)
constexpr int kCpOff = (kMaxE + 1 + 3) / 4 * 4;  // chunk prefix table, 16-byte aligned
constexpr int kTkOff = kCpOff + kMaxE + 1;     // work-ticket slots (2 words)
constexpr int kMatOff = kTkOff + 4;          // expert -> weight matrix table
constexpr int kTabInts = kMatOff + kMaxE;
constexpr int kPools = 8;                  // work-ticket counters per stage
constexpr int kUnit = 2;                   // consecutive items per ticket
#ifndef SMOE_FFN_STATIC_PERMILLE
#define SMOE_FFN_STATIC_PERMILLE 900
#endif
constexpr int kStaticPermille = SMOE_FFN_STATIC_PERMILLE;  // share of the even split taken up front
constexpr int kHdrStamp = 2;               // header words 2..5: the workspace stamp
constexpr int kHdrSpoiled = 6;             // header word 6: stamp mismatch seen
constexpr int kHdrCtr1 = 8;                // header words of the stage-1 counters
constexpr int kHdrCtr2 = kHdrCtr1 + kPools;
constexpr int kTabBytes = (kTabInts * 4 + 15) / 16 * 16;  // offsets, chunk prefix
static_assert(kTabBytes % 16 == 0, "staged rows must start 16-byte aligned");
constexpr int kMaxSlotsLds = 1024;         // sorted slots kept whole in LDS up to this many
constexpr int kLdsPerCu = 160 * 1024;      // gfx950
constexpr int kLdsBudget = kLdsPerCu / 2;  // per workgroup: two workgroups per CU
constexpr int kRowPad = 16;                // bytes of padding per staged row
#ifndef SMOE_FFN_D1
#define SMOE_FFN_D1 4
#endif
#ifndef SMOE_FFN_D2
#define SMOE_FFN_D2 3
#endif
constexpr int kD1 = SMOE_FFN_D1;           // blocks per item, stage 1 (8 KB per wave)
constexpr int kD2 = SMOE_FFN_D2;           // blocks per item, stage 2 (finer: fewer items per WG)
constexpr int kD1Narrow = 2;               // stage 1, INT4, NC = 2, x staged per item
constexpr int stage_d(int stage, int wk, int nc, int xres) {
  return stage == 2 ? kD2 : (wk == kInt4 && nc == 2 && !xres ? kD1Narrow : kD1);
}
// staged phases are whole INT4 items of the stage
constexpr int phase_k(int stage, int wk, int nc, int xres) {
  return stage_d(stage, wk, nc, xres) * 128;
}
#ifndef SMOE_FFN_MAX_WG
#define SMOE_FFN_MAX_WG 512
#endif
constexpr int kMaxWg = SMOE_FFN_MAX_WG;    // persistent grid cap
#ifndef SMOE_FFN_EXACT_SMALL
#define SMOE_FFN_EXACT_SMALL 1
#endif
constexpr bool kExactSmall = SMOE_FFN_EXACT_SMALL != 0;

// A set of experts that share a weight format and shapes: the routed
// experts (group 0) or the shared expert (group 1, FP16).
struct Group {
  const uint8_t* w0;            // stage 1: gate; stage 2: down
  const uint8_t* w1;            // stage 1: up
  const uint16_t* s0;           // INT4 group scales of w0 / w1 (fp16 bits)
  const uint16_t* s1;
  float* out;                   // stage 2 output [rows][H] (slot_out or shared_out)
  long long w_estride;          // bytes per expert
  long long s_estride;          // scale elements per expert
  long long gu_off;             // float offset of the group's g/u planes in a buffer
  int w_rstride;                // bytes per weight row
  int s_rstride;                // scale elements per row
  int fmt;                      // kInt4 or kFp16
  int tiled;                    // weights and scales in the 16-row tiled layout
  int N, K;                     // output rows and reduction length of this stage
  int nblk;                     // blocks per weight row
  int tiles, parts;             // row tiles and K parts per chunk
  int csz;                      // slots per chunk
  int rows;                     // slots of the group (S routed, T shared)
};

struct FfnArgs {
  const uint16_t* x;            // activations [T][H] (fp16 bits)
  const int32_t* sorted_slots;  // [S]
  const int32_t* offsets;       // [E+1]
  float* gu;                    // two g/u buffers
  int* hdr;                     // words 0, 1: call counter; then the work-ticket counters
                                // of stage 1 and of stage 2
  long long gu_buf;             // floats per g/u buffer
  int E, k, S, T, H;
  int chunks_upper;             // routed chunks the work list can hold
  int n_groups;                 // 1, or 2 with a shared expert
  int kph;                      // k per staged phase (a multiple of the stage's INT4 item)
  int stride;                   // LDS bytes per staged row
  int slots_lds;                // all S sorted slots copied to LDS at start
  int xs_off;                   // LDS byte offset of the staged rows
  int rows_lds;                 // staged rows the LDS holds (largest chunk)
  int xres;                     // stage 1: all T rows of x held in LDS for the whole launch
  Group grp[2];
  int has_mat;                  // mat holds the routed experts' weight matrices
  int32_t mat[kMaxE];           // matrix of expert e (-1: not in this call); else matrix e
};

// The launch's argument read in place from the kernel-argument segment (its
// only argument, at offset 0): indexing mat[] of the by-value argument with a
// run-time index would make the compiler copy the whole argument to scratch.
typedef const __attribute__((address_space(4))) FfnArgs ConstFfnArgs;
__device__ __forceinline__ ConstFfnArgs* ffn_kargs() {
  return (ConstFfnArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
}

// One item: part `part` of row tile `tile` of chunk `chunk` of group `grp`
// (expert e, positions [seg0, seg0 + m) of the group's slots).
struct Item {
  int grp, chunk, tile, part, e, me, seg0, m;  // me: weight matrix of expert e
};


template <int WK, int G, int STAGE, int NC, int XRES>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void ffn_kernel(
    FfnArgs a) {
  static_assert(XRES == 0 || STAGE == 1, "x is resident in stage 1 only");
  constexpr int D = stage_d(STAGE, WK, NC, XRES);
  constexpr int NQ = WK == kInt4 ? 128 / G : 1;  // INT4 group scales per block
  extern __shared__ __align__(16) uint8_t smem[];
  int* s_off = reinterpret_cast<int*>(smem);
  int* s_cp = s_off + kCpOff;
  int* s_tk = s_off + kTkOff;
  int* s_mat = s_off + kMatOff;
  int* s_slots = reinterpret_cast<int*>(smem + kTabBytes);  // all slots, or the chunk's
  uint8_t* xs = smem + a.xs_off;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int E = a.E;
  const int b = blockIdx.x;

  // ---- one round trip for the work list: expert offsets, sorted slots
  // (when they fit LDS) and the call counter
  static_assert(kThreads > kMaxE, "one offset per thread");
  const int offv = tid <= E ? a.offsets[tid] : 0;
  const int matv = a.has_mat && tid < E ? ffn_kargs()->mat[tid] : tid;
  constexpr int kSlotsPer = kMaxSlotsLds / kThreads;
  int slv[kSlotsPer];
  if (a.slots_lds) {
#pragma unroll
    for (int j = 0; j < kSlotsPer; ++j) {
      const int i = tid + j * kThreads;
      slv[j] = i < a.S ? a.sorted_slots[i] : -1;
    }
  }
  const int ep = a.hdr[STAGE == 1 ? 0 : 1];
  float* gu = a.gu + ((STAGE == 1 ? ep : ep - 1) & 1) * a.gu_buf;  // this call's g/u
  if (tid <= E) s_off[tid] = min(max(offv, 0), a.S);  // clamped to [0, S]
  if (a.has_mat && tid < E) s_mat[tid] = matv;
  // (stage 1 with x resident keeps the token of each sorted slot instead)
  constexpr bool xres = XRES != 0;
  if (a.slots_lds) {
#pragma unroll
    for (int j = 0; j < kSlotsPer; ++j)
      if (tid + j * kThreads < a.S)
        s_slots[tid + j * kThreads] =
            !xres ? slv[j] : (slv[j] >= 0 && slv[j] < a.S ? slv[j] / a.k : 0);
  }
  // Workspace stamp: the (T, k, I, shared I) the buffer serves, all zero on
  // a zeroed buffer. Stage 1 of the first call writes it; a call of another
  // shape marks the workspace spoiled (its g/u layout differs, so the
  // buffers no longer start at zero), and from then on stage 2 writes NaN
  // outputs instead of wrong sums, until the caller zeroes the buffer again.
  const int stamp_t = a.hdr[kHdrStamp], stamp_k = a.hdr[kHdrStamp + 1];
  const int stamp_i = a.hdr[kHdrStamp + 2], stamp_s = a.hdr[kHdrStamp + 3];
  const int spoiled = a.hdr[kHdrSpoiled];
  if (b == 0) {
    if (tid == 0) {
      a.hdr[STAGE == 1 ? 1 : 0] = STAGE == 1 ? ep + 1 : ep;
      if (STAGE == 1) {
        const int my_i = a.grp[0].N, my_s = a.n_groups > 1 ? a.grp[1].N : 0;
        if ((stamp_t | stamp_k | stamp_i | stamp_s) == 0) {
          a.hdr[kHdrStamp] = a.T;
          a.hdr[kHdrStamp + 1] = a.k;
          a.hdr[kHdrStamp + 2] = my_i;
          a.hdr[kHdrStamp + 3] = my_s;
        } else if (stamp_t != a.T || stamp_k != a.k || stamp_i != my_i || stamp_s != my_s) {
          a.hdr[kHdrSpoiled] = 1;
        }
      }
    }
    // the other stage's ticket counters start its next launch at zero
    if (tid < kPools)
      __hip_atomic_store(a.hdr + (STAGE == 1 ? kHdrCtr2 : kHdrCtr1) + tid, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (STAGE == 2 && spoiled) {
    // every output row NaN (this workgroup's share)
    const float qnan = __builtin_nanf("");
    const long long n_slot = static_cast<long long>(a.S) * a.H / 4;
    const long long tot = n_slot + (a.n_groups > 1 ? static_cast<long long>(a.T) * a.H / 4 : 0);
    for (long long i = static_cast<long long>(b) * kThreads + tid; i < tot;
         i += static_cast<long long>(gridDim.x) * kThreads) {
      f32x4* dst = i < n_slot ? reinterpret_cast<f32x4*>(a.grp[0].out) + i
                              : reinterpret_cast<f32x4*>(a.grp[1].out) + (i - n_slot);
      *dst = f32x4{qnan, qnan, qnan, qnan};
    }
    return;
  }

  // ---- work list: chunk prefix over the routed experts
  const int csz0 = a.grp[0].csz;
  if (wave == 0) {
    int n[4], tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      // (experts left out of the call have no chunks)
      n[i] = e < E && (!a.has_mat || s_mat[e] >= 0)
                 ? (max(s_off[e + 1] - s_off[e], 0) + csz0 - 1) / csz0 : 0;
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
  const int n_r = min(s_cp[E], a.chunks_upper) * a.grp[0].tiles * a.grp[0].parts;
  const int n_s = a.n_groups > 1
                      ? (a.T + a.grp[1].csz - 1) / a.grp[1].csz * a.grp[1].tiles * a.grp[1].parts
                      : 0;
  const int n_items = n_s + n_r;
  // Work split. Every workgroup first takes q0 consecutive items (nine
  // tenths of an even share, rounded down; none when that is under two).
  // The rest is cut into units of two consecutive items dealt out in
  // kPools pools:
  // pool p holds units p, p + kPools, ..., and workgroup b takes tickets
  // from the counter of pool b % kPools. A ticket for the unit that starts
  // at position pos + 2 of the workgroup's sequence is taken while it
  // works on position pos, so it is back long before it is needed. The
  // workgroups that stream faster take more units and all finish close
  // together.
  const int nwg = gridDim.x;
  int q0 = static_cast<int>(static_cast<long long>(n_items) * kStaticPermille / 1000 / nwg);
  int s0, dyn_base;
  if (q0 >= 2) {
    s0 = b * q0;
    dyn_base = nwg * q0;
  } else if (kExactSmall) {
    // A short list (under about two items per workgroup, as for a single
    // token): every item static, consecutive runs of n / nwg or one more, so
    // that no workgroup waits on a ticket before its first weight loads.
    const int base_q = n_items / nwg, extra = n_items - base_q * nwg;
    q0 = base_q + (b < extra ? 1 : 0);
    s0 = b * base_q + min(b, extra);
    dyn_base = n_items;
  } else {
    q0 = 0;
    s0 = 0;
    dyn_base = 0;
  }
  const int n_units = (n_items - dyn_base + kUnit - 1) / kUnit;
  const bool tickets = n_units > 0;
  const int pool = b & (kPools - 1);
  int* ctr = a.hdr + (STAGE == 1 ? kHdrCtr1 : kHdrCtr2) + pool;
  // first item of the unit of ticket t (-1: no such unit)
  auto unit_item = [&](int t) {
    const long long u = pool + static_cast<long long>(kPools) * t;
    return u < n_units ? dyn_base + kUnit * static_cast<int>(u) : -1;
  };
  // the item after `i` in its unit (-1 past the end of the list)
  auto next_in_unit = [&](int i) { return i >= 0 && i + 1 < n_items ? i + 1 : -1; };
  int cur, nxt;
  if (q0 > 0) {
    cur = s0;
    nxt = q0 > 1 ? s0 + 1 : -1;
  } else if (!tickets) {  // no items at all
    cur = nxt = -1;
  } else {  // no static run: tickets for positions 0 and 1 now
    if (tid == 0)
      s_tk[0] = __hip_atomic_fetch_add(ctr, kUnit > 1 ? 1 : 2, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int t = s_tk[0];
    cur = uniform(unit_item(t));
    nxt = uniform(kUnit > 1 ? next_in_unit(cur) : (cur >= 0 ? unit_item(t + 1) : -1));
    __syncthreads();  // the slot is free again
  }

  // Stage 1 clears what split tiles will add into: the stage-2 outputs and
  // the other g/u buffer (for the next call). Each workgroup clears its
  // share once its own items are done (or at once if it has none).
  auto clear_share = [&]() {
    if (STAGE != 1) return;
    float* other = a.gu + ((ep + 1) & 1) * a.gu_buf;
    const long long n0 = a.gu_buf / 4;
    // every row of slot_out, or with a matrix table only the rows of the
    // call's experts (below): the others keep what earlier calls wrote
    const long long n1 = n0 + (a.has_mat ? 0 : static_cast<long long>(a.S) * a.H / 4);
    const long long tot = n1 + (a.n_groups > 1 ? static_cast<long long>(a.T) * a.H / 4 : 0);
    const long long per = (tot + gridDim.x - 1) / gridDim.x;
    const long long lo = per * b, hi = min(tot, lo + per);
    for (long long i = lo + tid; i < hi; i += kThreads) {
      f32x4* dst = i < n0   ? reinterpret_cast<f32x4*>(other) + i
                   : i < n1 ? reinterpret_cast<f32x4*>(a.grp[0].out) + (i - n0)
                            : reinterpret_cast<f32x4*>(a.grp[1].out) + (i - n1);
      *dst = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if (a.has_mat) {
      const int kept = s_off[E];
      for (int p = b; p < kept; p += gridDim.x) {
        int lo_e = 0, hi_e = E;  // the expert of position p: s_off[lo_e] <= p < s_off[hi_e]
        while (hi_e - lo_e > 1) {
          const int mid = (lo_e + hi_e) >> 1;
          if (s_off[mid] <= p) lo_e = mid; else hi_e = mid;
        }
        const int row = a.sorted_slots[p];
        if (s_mat[lo_e] < 0 || row < 0 || row >= a.S) continue;
        f32x4* dst = reinterpret_cast<f32x4*>(a.grp[0].out) + static_cast<long long>(row) * (a.H / 4);
        for (int c = tid; c < a.H / 4; c += kThreads) dst[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  };
  if (cur < 0) {  // whole workgroup
    clear_share();
    return;
  }

  auto decode = [&](int item) {
    Item it;
    if (item >= n_s) {
      const int P = a.grp[0].parts, tiles = a.grp[0].tiles;
      const int ri = item - n_s;
      const int ct = ri / P;
      it.grp = 0;
      it.part = ri - ct * P;
      it.chunk = ct / tiles;
      it.tile = ct - it.chunk * tiles;
      // s_cp is non-decreasing, so the chunk's expert is the number of
      // experts whose chunks start at or before it, minus one
      const i32x4 cp = *reinterpret_cast<const i32x4*>(s_cp + 4 * lane);
      int n = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) n += __popcll(__ballot(4 * lane + i < E && cp[i] <= it.chunk));
      it.e = uniform(max(n - 1, 0));
      it.me = a.has_mat ? uniform(s_mat[it.e]) : it.e;
      it.seg0 = s_off[it.e] + (it.chunk - s_cp[it.e]) * csz0;
      it.m = min(csz0, s_off[it.e + 1] - it.seg0);
    } else {
      const int P = a.grp[1].parts, tiles = a.grp[1].tiles, csz = a.grp[1].csz;
      const int ct = item / P;
      it.grp = 1;
      it.part = item - ct * P;
      it.chunk = ct / tiles;
      it.tile = ct - it.chunk * tiles;
      it.e = 0;
      it.me = 0;
      it.seg0 = it.chunk * csz;
      it.m = min(csz, a.T - it.seg0);
    }
    return it;
  };

  // weight row of matrix m for this lane in row tile `tile`
  auto row_of = [&](int tile, int m) {
    return STAGE == 1 ? tile * (kWavesPerWg * 16) + wave * 16 + r16
                      : tile * (kWavesPerWg * 32) + wave * 32 + m * 16 + r16;
  };

  // ---- load cursor
  const uint8_t* wp[2];
  const uint16_t* sp[2];
  int l_blk0 = 0, l_nblk = 1, l_fmt = kFp16;
  // Tiled layout: the 16 rows of a wave's row slice and one block of k form
  // 1 KB in lane order (lane 16 g + r holds the 16 bytes that MFMA lane
  // group g of row r takes), so each load instruction reads 1 KB in one
  // piece; their scales form 16 NQ consecutive values. Row-major layout:
  // each lane reads within its own row.
  bool l_tiled = false;
  int l_bstride = kBlockBytes, l_sbstride = NQ;  // per block of k: bytes, scale elements
  auto set_load_item = [&](const Item& it) {
    const Group& gr = a.grp[it.grp];
    l_fmt = WK == kInt4 ? gr.fmt : kFp16;
    l_blk0 = it.part * D;
    l_nblk = gr.nblk;
    l_tiled = gr.tiled != 0;
    l_bstride = l_tiled ? 16 * kBlockBytes : kBlockBytes;
    l_sbstride = l_tiled ? 16 * NQ : NQ;
    const int lane_kb = (l_fmt == kInt4 && G == 64) ? 8 * g : (l_fmt == kInt4 && G == 32) ? 4 * g
                                                                                          : 16 * g;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t* wm = (STAGE == 1 && m == 1) ? gr.w1 : gr.w0;
      const uint16_t* sm = (STAGE == 1 && m == 1) ? gr.s1 : gr.s0;
      if (l_tiled) {
        // N is a multiple of 16: a slice past N is wholly past it, and
        // reads the last slice instead (loaded, never stored)
        const int sl = min(row_of(it.tile, m) >> 4, gr.N / 16 - 1);
        const long long t0 = static_cast<long long>(sl) * gr.nblk;
        wp[m] = wm + it.me * gr.w_estride + t0 * (16 * kBlockBytes) + 16 * lane;
        if (WK == kInt4) sp[m] = l_fmt == kInt4 ? sm + it.me * gr.s_estride + (t0 * 16 + r16) * NQ
                                                : sm;
      } else {
        const int row = min(row_of(it.tile, m), gr.N - 1);  // rows past N: loaded, never stored
        wp[m] = wm + it.me * gr.w_estride + static_cast<long long>(row) * gr.w_rstride + lane_kb;
        if (WK == kInt4)  // (FP16 groups: null + 0)
          sp[m] = sm + it.me * gr.s_estride + static_cast<long long>(row) * gr.s_rstride;
      }
    }
  };
  auto load = [&](u32x4 (&r)[2], int blk) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t* base = wp[m] + blk * l_bstride;
      if (WK == kInt4 && G != 128 && l_fmt == kInt4 && !l_tiled) {
        if (G == 64) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(base);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(base + 32);
          r[m] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            r[m][qq] = *reinterpret_cast<const uint32_t*>(base + 16 * qq);
        }
      } else {
        r[m] = *reinterpret_cast<const u32x4*>(base);
      }
    }
  };

  // INT4 group scales of an item, one load per matrix: lane group g holds
  // the scales of block blk0 + g of its row (NS words); block d reads them
  // from lane (d, row) with a cross-lane shuffle.
  static_assert(D <= 4, "one INT4 scale block per lane group");
  constexpr int NS = NQ == 4 ? 2 : 1;
  uint32_t sring[2][NS], scur[2][NS];
  auto load_scales = [&](int blk0) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint16_t* sptr = sp[m] + min(blk0 + g, l_nblk - 1) * l_sbstride;
      if (NQ == 1) {
        sring[m][0] = *sptr;
      } else if (NQ == 2) {
        sring[m][0] = *reinterpret_cast<const uint32_t*>(sptr);
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(sptr);
        sring[m][0] = v[0];
        sring[m][1] = v[1];
      }
    }
  };

  f32x4 acc[2][NC];
  uint32_t dq_lo = 0x000F000Fu, dq_hi = 0x00F000F0u, dq_magic = 0x64006400u;
  asm volatile("" : "+v"(dq_lo), "+v"(dq_hi), "+v"(dq_magic));  // keep the masks in VGPRs

  // Slot r of routed chunk `it` (from the full copy in LDS, or the chunk's copy).
  auto chunk_slot = [&](const Item& it, int r) {
    return a.slots_lds ? s_slots[it.seg0 + r] : s_slots[r];
  };
  // A operand rows (LDS byte offsets) of this lane; lanes past the chunk's
  // slots read a staged row and their results are dropped.
  int arow[NC];
#pragma unroll
  for (int cg = 0; cg < NC; ++cg) arow[cg] = min(16 * cg + r16, a.rows_lds - 1) * a.stride;

  // One INT4 block (128 k) at k offset kk of the staged rows.
  auto compute_int4 = [&](const u32x4 (&r)[2], int kk, int d, auto nce_tag) {
    constexpr int NCE = decltype(nce_tag)::value;
    constexpr int per = G / 32;
    f16x8 A[NCE == 1 ? 4 : 1];
    if (NCE == 1) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        A[qq] = *reinterpret_cast<const f16x8*>(xs + arow[0] + 2 * (kk + 8 * int4_word(G, g, qq)));
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      f16x8 B[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) B[qq] = dequant_word(r[m][qq], dq_lo, dq_hi, dq_magic);
#pragma unroll
      for (int grp = 0; grp < NQ; ++grp) {
        const int src = d * 16 + r16;
        const uint32_t word = __shfl(scur[m][NQ == 4 ? (grp >> 1) : 0], src, kWave);
        const uint32_t sbits = (NQ == 4) ? (word >> (16 * (grp & 1))) : (word >> (16 * grp));
        const float sc =
            static_cast<float>(bitcast<_Float16>(static_cast<uint16_t>(sbits & 0xFFFFu)));
#pragma unroll
        for (int cg = 0; cg < NCE; ++cg) {
          f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int qq = 0; qq < per; ++qq) {
            const int q = grp * per + qq;
            const f16x8 Aq = NCE == 1 ? A[q]
                                      : *reinterpret_cast<const f16x8*>(
                                            xs + arow[cg] + 2 * (kk + 8 * int4_word(G, g, q)));
            t = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aq, B[q], t, 0, 0, 0);
          }
          acc[m][cg] += sc * t;
          // one column group's operands in registers at a time
          if (NCE > 1) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  // One FP16 block (32 k) at k offset kk of the staged rows.
  // (resident x rows are k-permuted for row-major INT4 groups; the FP16
  // weights then take the same permutation. Tiled INT4 words dequantise in
  // natural k order, so with tiled weights nothing is permuted.)
  const bool xperm = WK == kInt4 && a.grp[0].tiled == 0;
  const bool bperm = xres && xperm;
  auto compute_fp16 = [&](const u32x4 (&r)[2], int kk, auto nce_tag) {
    constexpr int NCE = decltype(nce_tag)::value;
    f16x8 B[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) B[m] = bitcast<f16x8>(bperm ? permute_k8(r[m]) : r[m]);
#pragma unroll
    for (int cg = 0; cg < NCE; ++cg) {
      const f16x8 A = *reinterpret_cast<const f16x8*>(xs + arow[cg] + 2 * (kk + 8 * g));
#pragma unroll
      for (int m = 0; m < 2; ++m)
        acc[m][cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[m], acc[m][cg], 0, 0, 0);
    }
  };

  // Staged activations, eight k at a time: stage 1 copies x of the slot's
  // token; stage 2 forms fp16(SiLU(g) * u) of the position. The loads
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
      int tok = it.seg0 + r;  // shared expert: slot t is token t
      bool ok = true;
      if (it.grp == 0) {
        const int slot = chunk_slot(it, r);
        ok = slot >= 0 && slot < a.S;
        tok = ok ? slot / a.k : 0;
      }
      raw.v = *reinterpret_cast<const u32x4*>(a.x + static_cast<long long>(tok) * a.H + col);
      return ok;
    } else {
      const Group& gr = a.grp[it.grp];
      const float* gr_ = gu + gr.gu_off + static_cast<long long>(it.seg0 + r) * gr.K + col;
      const float* ur = gr_ + static_cast<long long>(gr.rows) * gr.K;
      raw.g0 = *reinterpret_cast<const f32x4*>(gr_);
      raw.g1 = *reinterpret_cast<const f32x4*>(gr_ + 4);
      raw.u0 = *reinterpret_cast<const f32x4*>(ur);
      raw.u1 = *reinterpret_cast<const f32x4*>(ur + 4);
      return true;
    }
  };
  auto finish = [&](const Raw& raw, bool perm) -> u32x4 {
    u32x4 v;
    if constexpr (STAGE == 1) {
      v = raw.v;
    } else {
      f16x8 h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = static_cast<_Float16>(raw.g0[i] / (1.0f + __expf(-raw.g0[i])) * raw.u0[i]);
        h[4 + i] = static_cast<_Float16>(raw.g1[i] / (1.0f + __expf(-raw.g1[i])) * raw.u1[i]);
      }
      v = bitcast<u32x4>(h);
    }
    return perm ? permute_k8(v) : v;
  };

  // Stage the activation rows of chunk `it`, k range [k0, k1), into
  // LDS. `mid` runs right after the first batch of loads is issued, so the
  // weight prologue can go out behind it without the staging waiting on it.
  auto stage_rows = [&](const Item& it, int k0, int k1, auto batch_tag, auto&& mid) {
    constexpr int NB = decltype(batch_tag)::value;  // pieces in flight per thread
    const Group& gr = a.grp[it.grp];
    __syncthreads();  // every wave is done with the previous rows
    if (!a.slots_lds && it.grp == 0) {
      if (tid < it.m) s_slots[tid] = a.sorted_slots[it.seg0 + tid];
      __syncthreads();
    }
    const bool perm = WK == kInt4 && gr.fmt == kInt4 && gr.tiled == 0;
    const int npr = (k1 - k0) / 8;  // 16-byte pieces per row
    const int tot = it.m * npr;
    for (int base = 0; base < tot; base += NB * kThreads) {
      Raw raw[NB];
      int dst[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int i = min(base + j * kThreads + tid, tot - 1);
        const int r = i / npr, c = i - r * npr;
        const bool ok = load_raw(it, r, k0 + 8 * c, raw[j]);
        dst[j] = (ok && base + j * kThreads + tid < tot) ? r * a.stride + 16 * c : -1;
      }
      if (base == 0) mid();
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (dst[j] >= 0) *reinterpret_cast<u32x4*>(xs + dst[j]) = finish(raw[j], perm);
    }
    __syncthreads();
  };

  // Stage 1 with x resident: all T rows of x, whole, once per launch (row t
  // at t * stride, k-permuted for INT4 weights), so no item restages.
  // `mid` runs right after the first batch of loads is issued; a batch
  // covers a 2048-wide window of 17 tokens, so at those sizes every x load
  // is out before the weight prologue and none waits behind it.
  auto stage_x_all = [&](auto&& mid) {
    constexpr int NB = 9;  // pieces in flight per thread
    const int npr = a.H / 8;
    const int tot = a.T * npr;
    for (int base = 0; base < tot; base += NB * kThreads) {
      u32x4 v[NB];
      int dst[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int i = min(base + j * kThreads + tid, tot - 1);
        const int r = i / npr, c = i - r * npr;
        v[j] = *reinterpret_cast<const u32x4*>(a.x + static_cast<long long>(r) * a.H + 8 * c);
        dst[j] = base + j * kThreads + tid < tot ? r * a.stride + 16 * c : -1;
      }
      if (base == 0) mid();
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (dst[j] >= 0)
          *reinterpret_cast<u32x4*>(xs + dst[j]) = xperm ? permute_k8(v[j]) : v[j];
    }
    __syncthreads();
  };

  // Write the sums of a tile; a tile split with other workgroups is added
  // into the (zeroed) output with device-scope atomics.
  auto write_tile = [&](const Item& it, bool whole) {
    const Group& gr = a.grp[it.grp];
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * cg + 4 * g + i;
        if (rr >= it.m) continue;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int row = row_of(it.tile, STAGE == 1 ? 0 : m);
          if (row >= gr.N) continue;
          float* dst;
          if (STAGE == 1) {
            dst = gu + gr.gu_off + static_cast<long long>(m) * gr.rows * gr.N +
                  static_cast<long long>(it.seg0 + rr) * gr.N + row;
          } else {
            int slot = it.seg0 + rr;  // shared expert: slot t is token t
            if (it.grp == 0) {
              slot = chunk_slot(it, rr);
              if (slot < 0 || slot >= a.S) continue;
            }
            dst = gr.out + static_cast<long long>(slot) * a.H + row;
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

  auto kblk_of = [&](int fmt) { return (WK == kInt4 && fmt == kInt4) ? 128 : 32; };
  // k window to stage for item `it` (number `item`), whose run of
  // consecutive items in this workgroup ends before run_end: if the run
  // stays in the item's tile, just the k it covers; else the LDS phase
  // holding the item (the rows then serve the next tiles of the chunk
  // too). At most kph wide.
  int st_lo = 0, st_hi = 0;
  auto window = [&](const Item& it, int item, int run_end) {
    const Group& gr = a.grp[it.grp];
    const int kpart = D * kblk_of(WK == kInt4 ? gr.fmt : kFp16);
    const int k0 = it.part * kpart;
    const int left_in_tile = gr.parts - 1 - it.part;  // items after this one in its tile
    if (run_end - 1 - item <= left_in_tile) {
      st_lo = k0;
      st_hi = min(gr.K, min(k0 + a.kph, (it.part + run_end - item) * kpart));
    } else {
      st_lo = k0 / a.kph * a.kph;
      st_hi = min(gr.K, st_lo + a.kph);
    }
  };
  // end of the run of consecutive items that `item` (at position pos) starts
  auto run_end_of = [&](int pos, int item, int next) {
    return pos < q0 ? s0 + q0 : (next == item + 1 ? item + 2 : item + 1);
  };

  // ---- prologue: stage the first chunk (or, x resident, all of x), the
  // first item's blocks in flight
  Item ci = decode(cur);
  set_load_item(ci);
  u32x4 ring[D][2];
  int c_fmt = l_fmt, c_nblk = l_nblk;
  int staged_id = ci.grp * (1 << 24) + ci.chunk;
  auto prologue_loads = [&]() {
    if (WK == kInt4 && l_fmt == kInt4) load_scales(l_blk0);
#pragma unroll
    for (int d = 0; d < D; ++d) load(ring[d], min(l_blk0 + d, l_nblk - 1));
  };
  if constexpr (xres) {
    st_lo = 0;
    st_hi = a.H;
    stage_x_all(prologue_loads);
  } else {
    window(ci, cur, run_end_of(0, cur, nxt));
    stage_rows(ci, st_lo, st_hi, std::integral_constant<int, STAGE == 1 ? 4 : 2>(),
               prologue_loads);
  }
  int seg_pa = ci.part;  // first part of the tile accumulated so far
  int prev = -2;         // the item before cur

  for (int pos = 0;; ++pos) {
    const int P = a.grp[ci.grp].parts;
    const int blk0 = ci.part * D;
    const int kblk = kblk_of(c_fmt);
    if (cur != prev + 1 || ci.part == 0) {
      seg_pa = ci.part;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) acc[m][cg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int id = ci.grp * (1 << 24) + ci.chunk;
    const int k0 = blk0 * kblk;
    const int k1 = min(a.grp[ci.grp].K, k0 + D * kblk);
    if constexpr (xres) {
      // A operand rows of this item: the tokens of its slots
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) {
        const int rr = max(min(16 * cg + r16, ci.m - 1), 0);
        const int tok = ci.grp == 0 ? s_slots[min(ci.seg0 + rr, a.S - 1)]
                                    : min(ci.seg0 + rr, a.T - 1);  // shared: slot t is token t
        arow[cg] = tok * a.stride;
      }
    } else if (id != staged_id || k0 < st_lo || k1 > st_hi) {
      window(ci, cur, run_end_of(pos, cur, nxt));
      stage_rows(ci, st_lo, st_hi, std::integral_constant<int, STAGE == 1 ? 2 : 1>(), []() {});
      staged_id = id;
    }

    // position pos + 2 starts a unit: take its ticket now
    const int r = pos + 2 - q0;
    const bool grab = tickets && r >= 0 && r % kUnit == 0 && nxt >= 0;
    int tk_new = 0;
    if (grab && tid == 0) {
      // the address goes through a VGPR so the compiler issues the plain
      // returning atomic (no cross-lane combining that waits on its result
      // right away); the result is first needed at the end of the item
      typedef __attribute__((address_space(1))) int global_int;
      global_int* cp = (global_int*)ctr;
      asm volatile("" : "+v"(cp));
      tk_new = __hip_atomic_fetch_add(cp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // the load cursor moves to the next item (or reloads this one's blocks)
    const bool l_live = nxt >= 0;
    if (WK == kInt4) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < NS; ++t) scur[m][t] = sring[m][t];
    }
    Item ni = ci;
    if (l_live) {
      ni = decode(nxt);
      set_load_item(ni);
      if (WK == kInt4 && l_fmt == kInt4) load_scales(l_blk0);
    }

    // (with x resident the routed chunks are at most 16 slots: only the
    // shared expert's chunks can be wide, and they are FP16)
    const bool wide = NC == 2 && ci.m > 16;
    const int kk0 = k0 - st_lo;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (blk0 + d < c_nblk) {
        if (WK == kInt4 && c_fmt == kInt4) {
          if (!xres && wide)
            compute_int4(ring[d], kk0 + d * 128, d, std::integral_constant<int, NC>());
          else
            compute_int4(ring[d], kk0 + d * 128, d, std::integral_constant<int, 1>());
        } else {
          if (wide)
            compute_fp16(ring[d], kk0 + d * 32, std::integral_constant<int, NC>());
          else
            compute_fp16(ring[d], kk0 + d * 32, std::integral_constant<int, 1>());
        }
      }
      load(ring[d], min(l_blk0 + d, l_nblk - 1));
    }

    if (nxt != cur + 1 || ci.part == P - 1) write_tile(ci, seg_pa == 0 && ci.part == P - 1);
    if (!l_live) break;
    if (grab) {
      if (tid == 0) s_tk[(r / kUnit) & 1] = tk_new;  // slots alternate between tickets
      __syncthreads();  // the new ticket is visible
    }
    int nn;
    if (r < 0)
      nn = s0 + pos + 2;
    else if (r % kUnit != 0)
      nn = tickets ? next_in_unit(nxt) : -1;
    else
      nn = tickets ? uniform(unit_item(s_tk[(r / kUnit) & 1])) : -1;
    prev = cur;
    cur = nxt;
    nxt = nn;
    ci = ni;
    c_fmt = l_fmt;
    c_nblk = l_nblk;
  }
  clear_share();
}

// Zero n16 16-byte words from p (the no-allocation entry point's workspace;
// a kernel rather than a memset so that the call stays graph-capturable).
__global__ __launch_bounds__(256) void zero_kernel(f32x4* __restrict__ p, long long n16) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += stride)
    p[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

}  // namespace
}  // namespace smoe

// Workspace of smoe_w4a16_expert_ffn_noalloc: one copy per device, held until
// the process ends. Host code never passes this name to a kernel (in host
// code it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device, in noalloc_scratch().
static __device__ __align__(256) uint8_t scratch[SMOE_NOALLOC_SCRATCH_BYTES];

namespace smoe {
namespace {

// Device address of `scratch` on the current device (looked up once per
// device with that device current), or null with the error text set.
void* noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("w4a16_expert_ffn_noalloc: no current device (or device index above %d)",
              kMaxDevices - 1);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr) {
      set_error("w4a16_expert_ffn_noalloc: hipGetSymbolAddress failed on device %d: %s", dev,
                hipGetErrorString(err));
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
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

// Slots per routed chunk: two 16-slot MFMA column groups when one expert is
// expected to hold more than 16 of the window's slots (long windows, or few
// experts), else one (an expert with more slots then gets a second chunk and
// reads its weights twice, which at these windows is rare).
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
// buffers, each [2][S][I] fp32 (routed) followed by [2][T][Is] fp32 (shared).
constexpr size_t kEpochBytes = 256;
long long gu_floats(long long T, long long k, long long I, long long Is) {
  return 2 * T * k * I + 2 * T * Is;
}
size_t gu_region_bytes(long long T, long long k, long long I, long long Is) {
  return kEpochBytes + static_cast<size_t>(2 * gu_floats(T, k, I, Is)) * sizeof(float);
}
// (long windows also keep the fp16 h of the long-window FFN after that,
// one-token windows the region of the single-token layer)
size_t workspace_bytes(long long T, long long k, long long H, long long I, long long Is) {
  const long long S = T * k;
  const bool wide = S >= kWideMinSlots && S <= kWideMaxSlots;
  return gu_region_bytes(T, k, I, Is) + (wide ? wide_h_bytes(T, k, I, Is) : 0) +
         (T == 1 ? decode_region_bytes(k, H, I, Is) : 0);
}


// Weights of one group as the entry points hand them over.
struct GroupWeights {
  int fmt;                       // kInt4 or kFp16
  int tiled;                     // 16-row tiled layout (else row-major)
  const void *wg, *wu, *wd;      // codes (INT4) or values (FP16)
  const void *sg, *su, *sd;      // INT4 scales, else null
  int E, I, G;                   // experts, intermediate size, INT4 group size
  int csz, rows;                 // slots per chunk, slots of the group
  float* out;                    // stage 2 output rows
  long long gu_off;              // float offset of its g/u planes
};

// Row geometry of a [E][N][K] weight tensor in the group's format.
void set_matrix(Group& g, const GroupWeights& w, int N, int K, const void* wq, const void* ws,
                int D) {
  g.fmt = w.fmt;
  g.tiled = w.tiled;
  g.N = N;
  g.K = K;
  g.w_rstride = w.fmt == kInt4 ? K / 2 : K * 2;
  g.w_estride = static_cast<long long>(g.w_rstride) * N;
  g.nblk = g.w_rstride / kBlockBytes;
  g.s_rstride = w.fmt == kInt4 ? K / w.G : 0;
  g.s_estride = static_cast<long long>(g.s_rstride) * N;
  g.w0 = static_cast<const uint8_t*>(wq);
  g.s0 = static_cast<const uint16_t*>(ws);
  g.parts = (g.nblk + D - 1) / D;
  g.csz = w.csz;
  g.rows = w.rows;
  g.out = w.out;
  g.gu_off = w.gu_off;
}

struct StagePlans {
  FfnArgs a1, a2;
  int lds1, lds2;
  long long items1, items2;  // upper bounds of the work lists
  int nc;
};

// LDS layout of a stage: the table, the sorted slots, then rows_lds staged
// rows of the phase length (a multiple of whole INT4 items, balanced over
// the phases that the longest K needs).
int xs_offset(long long S) {
  return kTabBytes + static_cast<int>(((S <= kMaxSlotsLds ? S : kMaxChunk) * 4 + 15) / 16 * 16);
}

int plan_lds(FfnArgs& a, int kmax, int kunit) {
  a.slots_lds = a.S <= kMaxSlotsLds ? 1 : 0;
  a.xs_off = xs_offset(a.S);
  const int per_row = (kLdsBudget - a.xs_off) / a.rows_lds;
  const int kph_cap = std::max(kunit, (per_row - kRowPad) / 2 / kunit * kunit);
  const int phases = (kmax + kph_cap - 1) / kph_cap;
  const int per_phase = (kmax + phases - 1) / phases;
  a.kph = (per_phase + kunit - 1) / kunit * kunit;
  a.stride = std::min(a.kph, kmax) * 2 + kRowPad;
  return a.xs_off + a.rows_lds * a.stride;
}

void make_plans(StagePlans& p, const void* x, int T, int k, int H, const int32_t* sorted_slots,
                const int32_t* offsets, void* workspace, const GroupWeights* gw, int n_groups) {
  const int S = T * k;
  uint8_t* wsb = static_cast<uint8_t*>(workspace);
  FfnArgs& a1 = p.a1;
  a1 = FfnArgs{};
  a1.x = static_cast<const uint16_t*>(x);
  a1.sorted_slots = sorted_slots;
  a1.offsets = offsets;
  a1.hdr = reinterpret_cast<int*>(wsb);
  a1.gu = reinterpret_cast<float*>(wsb + kEpochBytes);
  a1.gu_buf = gu_floats(T, k, gw[0].I, n_groups > 1 ? gw[1].I : 0);
  a1.E = gw[0].E; a1.k = k; a1.S = S; a1.T = T; a1.H = H;
  a1.chunks_upper = std::min(gw[0].E, S) + S / gw[0].csz;
  a1.n_groups = n_groups;
  a1.rows_lds = 1;
  for (int i = 0; i < n_groups; ++i) a1.rows_lds = std::max(a1.rows_lds, gw[i].csz);
  p.nc = a1.rows_lds > 16 ? 2 : 1;
  // stage 1 keeps all of x in LDS when it fits beside the table and the
  // sorted slots and the routed chunks are narrow: items then never restage
  // and the tail goes out one item at a time. Decided first: it sets the
  // stage-1 item size.
  const long long xres_bytes = xs_offset(S) + static_cast<long long>(T) * (2 * H + kRowPad);
  const bool xres = S <= kMaxSlotsLds && gw[0].csz <= 16 && xres_bytes <= kLdsBudget;
  const int d1 = stage_d(1, gw[0].fmt, p.nc, xres);
  FfnArgs& a2 = p.a2;
  a2 = a1;
  p.items1 = p.items2 = 0;
  int kmax2 = 0;
  for (int i = 0; i < n_groups; ++i) {
    const GroupWeights& w = gw[i];
    const long long chunks = i == 0 ? a1.chunks_upper : (T + w.csz - 1) / w.csz;
    set_matrix(a1.grp[i], w, w.I, H, w.wg, w.sg, d1);
    a1.grp[i].w1 = static_cast<const uint8_t*>(w.wu);
    a1.grp[i].s1 = static_cast<const uint16_t*>(w.su);
    a1.grp[i].tiles = tiles_of(w.I, 16);
    p.items1 += chunks * a1.grp[i].tiles * a1.grp[i].parts;
    set_matrix(a2.grp[i], w, H, w.I, w.wd, w.sd, stage_d(2, gw[0].fmt, p.nc, 0));
    a2.grp[i].w1 = nullptr;
    a2.grp[i].s1 = nullptr;
    a2.grp[i].tiles = tiles_of(H, 32);
    p.items2 += chunks * a2.grp[i].tiles * a2.grp[i].parts;
    kmax2 = std::max(kmax2, w.I);
  }
  p.lds1 = plan_lds(a1, H, phase_k(1, gw[0].fmt, p.nc, xres));
  p.lds2 = plan_lds(a2, kmax2, phase_k(2, gw[0].fmt, p.nc, 0));
  if (xres) {
    a1.xres = 1;
    a1.rows_lds = T;
    a1.kph = H;
    a1.stride = 2 * H + kRowPad;
    p.lds1 = static_cast<int>(xres_bytes);
  }
}

template <int WK, int G, int STAGE, int NC, int XRES>
smoe_status launch_stage(const FfnArgs& a, int lds, long long items, hipStream_t st) {
  auto kern = ffn_kernel<WK, G, STAGE, NC, XRES>;
  static std::atomic<int> attr_done{0};
  if (!attr_done.load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) != hipSuccess) {
      set_error("expert_ffn: cannot raise the dynamic LDS limit to %d bytes", kLdsBudget);
      return SMOE_EHIP;
    }
    attr_done.store(1, std::memory_order_release);
  }
  const int per_cu = 2 * lds <= kLdsPerCu ? 2 : 1;
  const long long cap = std::min<long long>(per_cu * cu_count(), kMaxWg);
  const int nwg = static_cast<int>(std::max(1ll, std::min(items, cap)));
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(kThreads), lds, st, a);
  return check_launch(STAGE == 1 ? "expert_ffn stage 1" : "expert_ffn stage 2");
}

template <int WK, int G, int NC>
smoe_status launch_ffn(const StagePlans& p, hipStream_t st) {
  smoe_status s = p.a1.xres ? launch_stage<WK, G, 1, NC, 1>(p.a1, p.lds1, p.items1, st)
                            : launch_stage<WK, G, 1, NC, 0>(p.a1, p.lds1, p.items1, st);
  if (s != SMOE_OK) return s;
  return launch_stage<WK, G, 2, NC, 0>(p.a2, p.lds2, p.items2, st);
}

smoe_status check_common(const char* who, const void* x, int T, int k, int E, int H, int I,
                         const int32_t* sorted_slots, const int32_t* offsets, int shared_I,
                         const void* swg, const void* swu, const void* swd, const void* workspace,
                         size_t ws_bytes, const float* slot_out, const float* shared_out) {
  SMOE_REQUIRE(T >= 0 && k > 0 && E > 0 && H > 0 && I > 0 && shared_I >= 0, SMOE_EINVAL,
               "%s: need T, shared_I >= 0 and k, E, H, I > 0 (T=%d k=%d E=%d H=%d I=%d "
               "shared_I=%d)", who, T, k, E, H, I, shared_I);
  // (k may exceed E here: a call can cover a subset of the experts, one of
  // them or one device's share, with the window's own k)
  SMOE_REQUIRE(E <= kMaxE && k <= kMaxK, SMOE_EUNSUPPORTED,
               "%s: need E <= 256 and k <= 8 (E=%d k=%d)", who, E, k);
  SMOE_REQUIRE(H % 128 == 0 && I % 128 == 0 && shared_I % 128 == 0, SMOE_EUNSUPPORTED,
               "%s: H, I and shared_I must be multiples of 128 (H=%d I=%d shared_I=%d)", who, H,
               I, shared_I);
  SMOE_REQUIRE(H <= 16384 && I <= 32768 && shared_I <= 32768, SMOE_EUNSUPPORTED,
               "%s: need H <= 16384 and I, shared_I <= 32768 (H=%d I=%d shared_I=%d)", who, H,
               I, shared_I);
  const long long S = static_cast<long long>(T) * k;
  SMOE_REQUIRE(S < (1ll << 24) && S * std::max(H, I) < (1ll << 31) &&
                   static_cast<long long>(T) * std::max(H, shared_I) < (1ll << 31),
               SMOE_EUNSUPPORTED,
               "%s: T*k must be below 2^24, T*k*max(H, I) and T*max(H, shared_I) below 2^31",
               who);
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(x && sorted_slots && offsets && workspace && slot_out, SMOE_EINVAL,
               "%s: null pointer", who);
  const size_t need = workspace_bytes(T, k, H, I, shared_I);
  SMOE_REQUIRE(ws_bytes >= need, SMOE_EINVAL, "%s: workspace of %zu bytes is below the %zu needed",
               who, ws_bytes, need);
  SMOE_REQUIRE(aligned16(x) && (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0 &&
                   aligned16(slot_out),
               SMOE_EINVAL,
               "%s: x and slot_out must be 16-byte aligned, the workspace 256-byte aligned", who);
  if (shared_I > 0) {
    SMOE_REQUIRE(swg && swu && swd && shared_out, SMOE_EINVAL,
                 "%s: null shared-expert pointer", who);
    SMOE_REQUIRE(aligned16(swg) && aligned16(swu) && aligned16(swd) && aligned16(shared_out),
                 SMOE_EINVAL, "%s: shared-expert weights and output must be 16-byte aligned",
                 who);
  }
  return SMOE_OK;
}

// Both groups as the entry points describe them; the work list must fit int.
smoe_status build_plans(const char* who, StagePlans& p, const void* x, int T, int k, int H,
                        const int32_t* sorted_slots, const int32_t* offsets, void* workspace,
                        GroupWeights routed, int shared_I, const void* swg, const void* swu,
                        const void* swd, float* slot_out, float* shared_out) {
  // (both groups share one layout; H, I and shared_I are multiples of 128)
  GroupWeights gw[2];
  routed.csz = chunk_slots(T, k, routed.E);
  routed.rows = T * k;
  routed.out = slot_out;
  routed.gu_off = 0;
  gw[0] = routed;
  int n = 1;
  if (shared_I > 0) {
    GroupWeights& s = gw[1];
    s = GroupWeights{};
    s.fmt = kFp16;
    s.tiled = routed.tiled;
    s.wg = swg; s.wu = swu; s.wd = swd;
    s.E = 1; s.I = shared_I; s.G = 0;
    s.csz = std::min(T, kMaxChunk);
    s.rows = T;
    s.out = shared_out;
    s.gu_off = 2ll * T * k * routed.I;
    n = 2;
  }
  make_plans(p, x, T, k, H, sorted_slots, offsets, workspace, gw, n);
  SMOE_REQUIRE(p.lds1 <= kLdsBudget && p.lds2 <= kLdsBudget, SMOE_EUNSUPPORTED,
               "%s: staged rows need %d / %d bytes of LDS, above %d", who, p.lds1, p.lds2,
               kLdsBudget);
  SMOE_REQUIRE(p.items1 < (1ll << 31) && p.items2 < (1ll << 31), SMOE_EUNSUPPORTED,
               "%s: the work list exceeds 2^31 items (T=%d k=%d H=%d)", who, T, k, H);
  return SMOE_OK;
}

// Tiled weights and a long window: the long-window FFN (ffn_wide.hip), whose
// fp16 h lives after the g/u region of the workspace. Returns false (nothing
// enqueued) when it does not apply.
bool try_wide(smoe_status& st, const char* who, const GroupWeights& r, const void* x, int T,
              int k, int H, const int32_t* sorted_slots, const int32_t* offsets, int shared_I,
              const void* swg, const void* swu, const void* swd, void* workspace,
              float* slot_out, float* shared_out, hipStream_t s) {
  if (!r.tiled) return false;
  WideCall c{};
  c.fmt = r.fmt;
  c.G = r.G;
  c.x = x;
  c.T = T; c.k = k; c.E = r.E; c.H = H; c.I = r.I;
  c.wg = r.wg; c.wu = r.wu; c.wd = r.wd;
  c.sg = r.sg; c.su = r.su; c.sd = r.sd;
  c.Is = shared_I;
  c.swg = swg; c.swu = swu; c.swd = swd;
  c.sorted_slots = sorted_slots;
  c.offsets = offsets;
  c.h = static_cast<uint8_t*>(workspace) + gu_region_bytes(T, k, r.I, shared_I);
  c.slot_out = slot_out;
  c.shared_out = shared_I > 0 ? shared_out : nullptr;
  if (!wide_applicable(c)) return false;
  st = wide_ffn(c, s, who);
  return true;
}

// clear_ws: zero the workspace bytes this call uses before its launches
// (the no-allocation entry point, whose workspace other calls share).
smoe_status w4a16_ffn(int tiled,
    const void* x, int T, int k, int E, int H, int I, int group_size, const uint32_t* wg_q,
    const void* wg_s, const uint32_t* wu_q, const void* wu_s, const uint32_t* wd_q,
    const void* wd_s, const int32_t* sorted_slots, const int32_t* expert_offsets, int shared_I,
    const void* shared_wg, const void* shared_wu, const void* shared_wd, void* workspace,
    size_t workspace_bytes_, float* slot_out, float* shared_out, void* stream,
    bool clear_ws = false, const char* who = nullptr) {
  if (who == nullptr) who = tiled ? "w4a16_expert_ffn_tiled" : "w4a16_expert_ffn";
  SMOE_REQUIRE(group_size == 32 || group_size == 64 || group_size == 128, SMOE_EUNSUPPORTED,
               "%s: group size must be 32, 64 or 128 (got %d)", who, group_size);
  smoe_status st = check_common(who, x, T, k, E, H, I, sorted_slots, expert_offsets, shared_I,
                                shared_wg, shared_wu, shared_wd, workspace, workspace_bytes_,
                                slot_out, shared_out);
  if (st != SMOE_OK) return st;
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(wg_q && wg_s && wu_q && wu_s && wd_q && wd_s, SMOE_EINVAL,
               "%s: null weight pointer", who);
  SMOE_REQUIRE(aligned16(wg_q) && aligned16(wu_q) && aligned16(wd_q), SMOE_EINVAL,
               "%s: packed weights must be 16-byte aligned", who);
  SMOE_REQUIRE(((reinterpret_cast<uintptr_t>(wg_s) | reinterpret_cast<uintptr_t>(wu_s) |
                 reinterpret_cast<uintptr_t>(wd_s)) & 7u) == 0,
               SMOE_EINVAL, "%s: scales must be 8-byte aligned", who);

  GroupWeights r{};
  r.fmt = kInt4;
  r.tiled = tiled;
  r.wg = wg_q; r.wu = wu_q; r.wd = wd_q;
  r.sg = wg_s; r.su = wu_s; r.sd = wd_s;
  r.E = E; r.I = I; r.G = group_size;
  StagePlans p;
  st = build_plans(who, p, x, T, k, H, sorted_slots, expert_offsets, workspace, r, shared_I,
                   shared_wg, shared_wu, shared_wd, slot_out, shared_out);
  if (st != SMOE_OK) return st;
  hipStream_t s = as_stream(stream);
  if (try_wide(st, who, r, x, T, k, H, sorted_slots, expert_offsets, shared_I, shared_wg,
               shared_wu, shared_wd, workspace, slot_out, shared_out, s))
    return st;
  if (clear_ws) {
    const long long n16 = static_cast<long long>(gu_region_bytes(T, k, I, shared_I) / 16);
    const int grid = static_cast<int>(std::min<long long>((n16 + 255) / 256, 2048));
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s,
                       static_cast<f32x4*>(workspace), n16);
    st = check_launch(who);
    if (st != SMOE_OK) return st;
  }
#define SMOE_FFN_NC(G) \
  (p.nc == 2 ? launch_ffn<kInt4, G, 2>(p, s) : launch_ffn<kInt4, G, 1>(p, s))
  switch (group_size) {
    case 32: return SMOE_FFN_NC(32);
    case 64: return SMOE_FFN_NC(64);
    default: return SMOE_FFN_NC(128);
  }
#undef SMOE_FFN_NC
}

// mat / n_mat: the expert -> weight matrix table of smoe_fp16_expert_ffn_mapped
// (null: expert e is matrix e).
smoe_status fp16_ffn(int tiled,
    const void* x, int T, int k, int E, int H, int I, const void* wg, const void* wu,
    const void* wd, const int32_t* sorted_slots, const int32_t* expert_offsets, int shared_I,
    const void* shared_wg, const void* shared_wu, const void* shared_wd, void* workspace,
    size_t workspace_bytes_, float* slot_out, float* shared_out, void* stream,
    const int32_t* mat = nullptr, int n_mat = 0, const char* who = nullptr) {
  if (who == nullptr) who = tiled ? "fp16_expert_ffn_tiled" : "fp16_expert_ffn";
  smoe_status st = check_common(who, x, T, k, E, H, I, sorted_slots, expert_offsets, shared_I,
                                shared_wg, shared_wu, shared_wd, workspace, workspace_bytes_,
                                slot_out, shared_out);
  if (st != SMOE_OK) return st;
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(wg && wu && wd, SMOE_EINVAL, "%s: null weight pointer", who);
  SMOE_REQUIRE(aligned16(wg) && aligned16(wu) && aligned16(wd), SMOE_EINVAL,
               "%s: weights must be 16-byte aligned", who);
  GroupWeights r{};
  r.fmt = kFp16;
  r.tiled = tiled;
  r.wg = wg; r.wu = wu; r.wd = wd;
  r.E = E; r.I = I; r.G = 0;
  StagePlans p;
  st = build_plans(who, p, x, T, k, H, sorted_slots, expert_offsets, workspace, r, shared_I,
                   shared_wg, shared_wu, shared_wd, slot_out, shared_out);
  if (st != SMOE_OK) return st;
  if (mat != nullptr) {  // (host table; an index outside the arrays leaves the expert out)
    p.a1.has_mat = p.a2.has_mat = 1;
    for (int e = 0; e < E; ++e)
      p.a1.mat[e] = p.a2.mat[e] = mat[e] >= 0 && mat[e] < n_mat ? mat[e] : -1;
  }
  hipStream_t s = as_stream(stream);
  if (mat == nullptr &&
      try_wide(st, who, r, x, T, k, H, sorted_slots, expert_offsets, shared_I, shared_wg,
               shared_wu, shared_wd, workspace, slot_out, shared_out, s))
    return st;
  return p.nc == 2 ? launch_ffn<kFp16, 128, 2>(p, s) : launch_ffn<kFp16, 128, 1>(p, s);
}

smoe_status moe_layer(int tiled,
    const void* x, const float* w_router, const float* logit_bias, int T, int H, int E, int k,
    int flags, int32_t* topk_ids, float* topk_w, float* logits, const float* shared_gate_w,
    float* shared_gate, int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
    int32_t* active_experts, int32_t* n_active, int32_t* elb_counts, int L, int layer, int M,
    int32_t* plan_ids, int32_t* plan_counts, int elb_flags, int I, int group_size,
    const uint32_t* wg_q, const void* wg_s, const uint32_t* wu_q, const void* wu_s,
    const uint32_t* wd_q, const void* wd_s, int shared_I, const void* shared_wg,
    const void* shared_wu, const void* shared_wd, void* workspace, size_t workspace_bytes_,
    float* slot_out, float* shared_out, void* y, void* stream) {
  const char* who = tiled ? "moe_layer_w4a16_tiled" : "moe_layer_w4a16";
  // every step's checks before anything is enqueued
  RouteArgs ra;
  smoe_status st = route_check(x, w_router, logit_bias, T, H, E, k, flags, topk_ids, topk_w,
                               logits, shared_gate_w, shared_gate, ra);
  if (st != SMOE_OK) return st;
  st = align_check(topk_ids, T, k, E, expert_counts, expert_offsets, sorted_slots,
                   active_experts, n_active);
  if (st != SMOE_OK) return st;
  if (elb_counts != nullptr) {
    st = elb_check(elb_counts, L, E, topk_ids, layer, 1, T, k, M, plan_ids, elb_flags);
    if (st != SMOE_OK) return st;
  }
  SMOE_REQUIRE(group_size == 32 || group_size == 64 || group_size == 128, SMOE_EUNSUPPORTED,
               "%s: group size must be 32, 64 or 128 (got %d)", who, group_size);
  st = check_common(who, x, T, k, E, H, I, sorted_slots, expert_offsets, shared_I, shared_wg,
                    shared_wu, shared_wd, workspace, workspace_bytes_, slot_out, shared_out);
  if (st != SMOE_OK) return st;
  const float* s_out = shared_I > 0 ? shared_out : nullptr;
  st = combine_check(slot_out, topk_w, T, k, H, s_out, shared_gate, y);
  if (st != SMOE_OK) return st;
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(wg_q && wg_s && wu_q && wu_s && wd_q && wd_s, SMOE_EINVAL,
               "%s: null weight pointer", who);
  SMOE_REQUIRE(aligned16(wg_q) && aligned16(wu_q) && aligned16(wd_q), SMOE_EINVAL,
               "%s: packed weights must be 16-byte aligned", who);
  SMOE_REQUIRE(((reinterpret_cast<uintptr_t>(wg_s) | reinterpret_cast<uintptr_t>(wu_s) |
                 reinterpret_cast<uintptr_t>(wd_s)) & 7u) == 0,
               SMOE_EINVAL, "%s: scales must be 8-byte aligned", who);
  GroupWeights r{};
  r.fmt = kInt4;
  r.tiled = tiled;
  r.wg = wg_q; r.wu = wu_q; r.wd = wd_q;
  r.sg = wg_s; r.su = wu_s; r.sd = wd_s;
  r.E = E; r.I = I; r.G = group_size;
  StagePlans p;
  st = build_plans(who, p, x, T, k, H, sorted_slots, expert_offsets, workspace, r, shared_I,
                   shared_wg, shared_wu, shared_wd, slot_out, shared_out);
  if (st != SMOE_OK) return st;
  if (tiled && decode_applicable(T, k, E, H, I, shared_I, group_size)) {
    // one token: the single-token layer, two launches with the routing
    // inside the first (same outputs as the steps below)
    DecodeCall c{};
    c.f.r = ra;
    c.f.counts = expert_counts;
    c.f.offsets = expert_offsets;
    c.f.sorted_slots = sorted_slots;
    c.f.active = active_experts;
    c.f.n_active = n_active;
    c.f.elb_counts = elb_counts;
    c.f.plan_ids = plan_ids;
    c.f.plan_counts = plan_counts;
    c.f.L = L;
    c.f.layer = layer;
    c.f.M = elb_counts != nullptr ? M : 0;
    c.f.elb_clear = (elb_flags & SMOE_ELB_CLEAR_AFTER) ? 1 : 0;
    c.G = group_size;
    c.I = I;
    c.Is = shared_I;
    c.wg = wg_q; c.wu = wu_q; c.wd = wd_q;
    c.sg = wg_s; c.su = wu_s; c.sd = wd_s;
    c.swg = shared_wg; c.swu = shared_wu; c.swd = shared_wd;
    c.region = static_cast<uint8_t*>(workspace) + gu_region_bytes(T, k, I, shared_I);
    c.slot_out = slot_out;
    c.shared_out = shared_I > 0 ? shared_out : nullptr;
    c.y = y;
    return decode_layer(c, as_stream(stream), who);
  }
  // (the steps' own checks pass again; they enqueue the launches)
  // The shared experts' weights (every layout holds shared_I * H FP16
  // values per matrix) are read through the caches by the rest of the
  // routing launch, one workgroup per remaining CU (fewer cannot read them
  // within the routing's time), when they fit in what HBM moves during the
  // routing of a short window: DeepSeek-V2-Lite's 34.6 MB made its layer
  // 93.4 against 95.2 us; Qwen1.5-MoE's 69 MB made the routing launch
  // 13.7 against 6.2 us and the layer 7 us slower.
  RoutePrefetch pf{};
  constexpr long long kPrefetchMaxBytes = 40ll << 20;
  if (shared_I > 0 && 3 * 2ll * shared_I * H <= kPrefetchMaxBytes) {
    const long long mb = 2ll * shared_I * H;
    pf.p[0] = shared_wg; pf.bytes[0] = mb;
    pf.p[1] = shared_wu; pf.bytes[1] = mb;
    pf.p[2] = shared_wd; pf.bytes[2] = mb;
    pf.wgs = std::max(1, cu_count() - 1);
  }
  st = route_align_elb(x, w_router, logit_bias, T, H, E, k, flags, topk_ids, topk_w, logits,
                       shared_gate_w, shared_gate, expert_counts, expert_offsets, sorted_slots,
                       active_experts, n_active, elb_counts, L, layer, M, plan_ids, plan_counts,
                       elb_flags, stream, &pf);
  if (st != SMOE_OK) return st;
  st = w4a16_ffn(tiled, x, T, k, E, H, I, group_size, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s,
                             sorted_slots, expert_offsets, shared_I, shared_wg, shared_wu,
                             shared_wd, workspace, workspace_bytes_, slot_out, shared_out, stream);
  if (st != SMOE_OK) return st;
  return smoe_combine(slot_out, topk_w, T, k, H, s_out, shared_gate, y, stream);
}

}  // namespace
}  // namespace smoe

using namespace smoe;

extern "C" size_t smoe_ffn_workspace_bytes(int T, int k, int E, int H, int I, int shared_I) {
  if (T <= 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0 || shared_I < 0) return 0;
  return workspace_bytes(T, k, H, I, shared_I);
}

extern "C" smoe_status smoe_w4a16_expert_ffn(
    const void* x, int T, int k, int E, int H, int I, int group_size, const uint32_t* wg_q,
    const void* wg_s, const uint32_t* wu_q, const void* wu_s, const uint32_t* wd_q,
    const void* wd_s, const int32_t* sorted_slots, const int32_t* expert_offsets, int shared_I,
    const void* shared_wg, const void* shared_wu, const void* shared_wd, void* workspace,
    size_t workspace_bytes_, float* slot_out, float* shared_out, void* stream) {
  clear_error();
  return w4a16_ffn(0, x, T, k, E, H, I, group_size, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, sorted_slots,
                   expert_offsets, shared_I, shared_wg, shared_wu, shared_wd, workspace,
                   workspace_bytes_, slot_out, shared_out, stream);
}

extern "C" smoe_status smoe_w4a16_expert_ffn_noalloc(
    const void* x, int T, int k, int E, int H, int I, int group_size, const uint32_t* wg_q,
    const void* wg_s, const uint32_t* wu_q, const void* wu_s, const uint32_t* wd_q,
    const void* wd_s, const int32_t* sorted_slots, const int32_t* expert_offsets, int shared_I,
    const void* shared_wg, const void* shared_wu, const void* shared_wd, float* slot_out,
    float* shared_out, void* stream) {
  clear_error();
  const char* who = "w4a16_expert_ffn_noalloc";
  SMOE_REQUIRE(group_size == 32 || group_size == 64 || group_size == 128, SMOE_EUNSUPPORTED,
               "%s: group size must be 32, 64 or 128 (got %d)", who, group_size);
  // the size limit first: it needs no device
  if (T > 0 && k > 0 && E > 0 && H > 0 && I > 0 && shared_I >= 0) {
    const size_t need = workspace_bytes(T, k, H, I, shared_I);
    SMOE_REQUIRE(need <= SMOE_NOALLOC_SCRATCH_BYTES, SMOE_EUNSUPPORTED,
                 "%s: the window needs %zu bytes of workspace, above the %zu bytes of the "
                 "library's static workspace (T=%d k=%d I=%d shared_I=%d); use "
                 "smoe_w4a16_expert_ffn with a workspace of that size",
                 who, need, static_cast<size_t>(SMOE_NOALLOC_SCRATCH_BYTES), T, k, I, shared_I);
  }
  // every other check on host values before the device is touched
  smoe_status st = check_common(who, x, T, k, E, H, I, sorted_slots, expert_offsets, shared_I,
                                shared_wg, shared_wu, shared_wd, reinterpret_cast<void*>(256),
                                SMOE_NOALLOC_SCRATCH_BYTES, slot_out, shared_out);
  if (st != SMOE_OK || T == 0) return st;
  void* ws = noalloc_scratch();
  if (ws == nullptr) return SMOE_EHIP;
  return w4a16_ffn(0, x, T, k, E, H, I, group_size, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s,
                   sorted_slots, expert_offsets, shared_I, shared_wg, shared_wu, shared_wd, ws,
                   SMOE_NOALLOC_SCRATCH_BYTES, slot_out, shared_out, stream, /*clear_ws=*/true,
                   who);
}

extern "C" smoe_status smoe_w4a16_expert_ffn_tiled(
    const void* x, int T, int k, int E, int H, int I, int group_size, const uint32_t* wg_q,
    const void* wg_s, const uint32_t* wu_q, const void* wu_s, const uint32_t* wd_q,
    const void* wd_s, const int32_t* sorted_slots, const int32_t* expert_offsets, int shared_I,
    const void* shared_wg, const void* shared_wu, const void* shared_wd, void* workspace,
    size_t workspace_bytes_, float* slot_out, float* shared_out, void* stream) {
  clear_error();
  return w4a16_ffn(1, x, T, k, E, H, I, group_size, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, sorted_slots,
                   expert_offsets, shared_I, shared_wg, shared_wu, shared_wd, workspace,
                   workspace_bytes_, slot_out, shared_out, stream);
}

extern "C" smoe_status smoe_fp16_expert_ffn(
    const void* x, int T, int k, int E, int H, int I, const void* wg, const void* wu,
    const void* wd, const int32_t* sorted_slots, const int32_t* expert_offsets, int shared_I,
    const void* shared_wg, const void* shared_wu, const void* shared_wd, void* workspace,
    size_t workspace_bytes_, float* slot_out, float* shared_out, void* stream) {
  clear_error();
  return fp16_ffn(0, x, T, k, E, H, I, wg, wu, wd, sorted_slots, expert_offsets, shared_I, shared_wg,
                  shared_wu, shared_wd, workspace, workspace_bytes_, slot_out, shared_out, stream);
}

extern "C" smoe_status smoe_fp16_expert_ffn_tiled(
    const void* x, int T, int k, int E, int H, int I, const void* wg, const void* wu,
    const void* wd, const int32_t* sorted_slots, const int32_t* expert_offsets, int shared_I,
    const void* shared_wg, const void* shared_wu, const void* shared_wd, void* workspace,
    size_t workspace_bytes_, float* slot_out, float* shared_out, void* stream) {
  clear_error();
  return fp16_ffn(1, x, T, k, E, H, I, wg, wu, wd, sorted_slots, expert_offsets, shared_I, shared_wg,
                  shared_wu, shared_wd, workspace, workspace_bytes_, slot_out, shared_out, stream);
}

extern "C" smoe_status smoe_fp16_expert_ffn_mapped(
    const void* x, int T, int k, int E, int H, int I, const void* wg, const void* wu,
    const void* wd, int tiled, int n_matrices, const int32_t* expert_matrix,
    const int32_t* sorted_slots, const int32_t* expert_offsets, int shared_I,
    const void* shared_wg, const void* shared_wu, const void* shared_wd, void* workspace,
    size_t workspace_bytes_, float* slot_out, float* shared_out, void* stream) {
  clear_error();
  const char* who = "fp16_expert_ffn_mapped";
  SMOE_REQUIRE(tiled == 0 || tiled == 1, SMOE_EINVAL, "%s: tiled must be 0 or 1 (got %d)", who,
               tiled);
  SMOE_REQUIRE(n_matrices > 0, SMOE_EINVAL, "%s: need n_matrices > 0 (got %d)", who,
               n_matrices);
  SMOE_REQUIRE(T == 0 || expert_matrix != nullptr, SMOE_EINVAL, "%s: null expert_matrix", who);
  return fp16_ffn(tiled, x, T, k, E, H, I, wg, wu, wd, sorted_slots, expert_offsets, shared_I,
                  shared_wg, shared_wu, shared_wd, workspace, workspace_bytes_, slot_out,
                  shared_out, stream, expert_matrix, n_matrices, who);
}

extern "C" smoe_status smoe_ffn_workspace_clear(void* workspace, size_t workspace_bytes_,
                                                void* stream) {
  clear_error();
  SMOE_REQUIRE(workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0,
               SMOE_EINVAL, "ffn_workspace_clear: the workspace must be non-null and 256-byte "
               "aligned");
  SMOE_REQUIRE(workspace_bytes_ % 16 == 0, SMOE_EINVAL,
               "ffn_workspace_clear: workspace_bytes must be a multiple of 16 (got %zu)",
               workspace_bytes_);
  if (workspace_bytes_ == 0) return SMOE_OK;
  const long long n16 = static_cast<long long>(workspace_bytes_ / 16);
  const int grid = static_cast<int>(std::min<long long>((n16 + 255) / 256, 2048));
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, as_stream(stream),
                     static_cast<f32x4*>(workspace), n16);
  return check_launch("ffn_workspace_clear");
}

extern "C" smoe_status smoe_moe_layer_w4a16(
    const void* x, const float* w_router, const float* logit_bias, int T, int H, int E, int k,
    int flags, int32_t* topk_ids, float* topk_w, float* logits, const float* shared_gate_w,
    float* shared_gate, int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
    int32_t* active_experts, int32_t* n_active, int32_t* elb_counts, int L, int layer, int M,
    int32_t* plan_ids, int32_t* plan_counts, int elb_flags, int I, int group_size,
    const uint32_t* wg_q, const void* wg_s, const uint32_t* wu_q, const void* wu_s,
    const uint32_t* wd_q, const void* wd_s, int shared_I, const void* shared_wg,
    const void* shared_wu, const void* shared_wd, void* workspace, size_t workspace_bytes_,
    float* slot_out, float* shared_out, void* y, void* stream) {
  clear_error();
  return moe_layer(0, x, w_router, logit_bias, T, H, E, k, flags, topk_ids, topk_w, logits,
                   shared_gate_w, shared_gate, expert_counts, expert_offsets, sorted_slots,
                   active_experts, n_active, elb_counts, L, layer, M, plan_ids, plan_counts,
                   elb_flags, I, group_size, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, shared_I,
                   shared_wg, shared_wu, shared_wd, workspace, workspace_bytes_, slot_out,
                   shared_out, y, stream);
}

extern "C" smoe_status smoe_moe_layer_w4a16_tiled(
    const void* x, const float* w_router, const float* logit_bias, int T, int H, int E, int k,
    int flags, int32_t* topk_ids, float* topk_w, float* logits, const float* shared_gate_w,
    float* shared_gate, int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
    int32_t* active_experts, int32_t* n_active, int32_t* elb_counts, int L, int layer, int M,
    int32_t* plan_ids, int32_t* plan_counts, int elb_flags, int I, int group_size,
    const uint32_t* wg_q, const void* wg_s, const uint32_t* wu_q, const void* wu_s,
    const uint32_t* wd_q, const void* wd_s, int shared_I, const void* shared_wg,
    const void* shared_wu, const void* shared_wd, void* workspace, size_t workspace_bytes_,
    float* slot_out, float* shared_out, void* y, void* stream) {
  clear_error();
  return moe_layer(1, x, w_router, logit_bias, T, H, E, k, flags, topk_ids, topk_w, logits,
                   shared_gate_w, shared_gate, expert_counts, expert_offsets, sorted_slots,
                   active_experts, n_active, elb_counts, L, layer, M, plan_ids, plan_counts,
                   elb_flags, I, group_size, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, shared_I,
                   shared_wg, shared_wu, shared_wd, workspace, workspace_bytes_, slot_out,
                   shared_out, y, stream);
}
