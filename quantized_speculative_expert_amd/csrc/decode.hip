// Single-token draft layer over tiled weights: the whole MoE layer of one
// autoregressive draft token (router, top-k, alignment, ELB update, the
// routed W4A16 experts, the FP16 shared experts and the combine) in two
// launches.
//
// Specter paper: fused multi-expert draft kernel paragraph (one launch over
// every active expert, to amortise launch latency when the draft runs one
// token at a time), State Manager paragraph (the draft is autoregressive),
// Incremental Routing Pattern Analyzer paragraphs (the draft router's top-k
// IDs counted per layer, ranked top-M), hybrid-precision layout (INT4
// routed experts, FP16 shared experts, full-precision router). Design
// notes, "Streamlined Execution Engine" (INT4 tiles dequantised in the
// kernel, FP16 activations, FP32 sums).
//
// With one token every weight byte meets one activation: the layer is a
// stream of 60 MB of weights (DeepSeek-V2-Lite shape), and what decides its
// time is how soon the bytes start flowing, not the arithmetic. So:
//   launch 1  router rows | shared gate/up | routed gate/up
//     - the first workgroups compute the router rows and publish them;
//       workgroup 0 then gathers them and runs the top-k, the alignment
//       and the ELB update (the same block as smoe_route_align_elb) for
//       the call's outputs;
//     - the shared experts need no routing: their workgroups stream as soon
//       as the router rows are out (so that the rows' loads do not queue
//       behind the stream), while the routed workgroups take the top-k;
//     - each routed workgroup loads its activations, gathers the published
//       router rows and takes the top-k itself (the same wave routine as
//       the routing calls, so the same experts), then streams two 16-row
//       slabs of its slot's expert.
//     Each workgroup takes its slabs of gate and up over the whole K (its
//     eight waves split the blocks, partial sums meet in LDS), so
//     SiLU(g) * u is formed once, rounded to fp16 like the other FFN paths.
//   launch 2  down + combine
//     A workgroup takes one 16-row slab of the output and one routed slot,
//     or half of the shared expert's K (every workgroup of the launch is
//     resident at once). The slab's last workgroup gathers the other parts
//     and writes slot_out, shared_out and y = fp16(sum_j w_j out_j +
//     gate * shared) in the combine's order.
// No dot product is split by timing: the results are the same on every run.
//
// Values pass between workgroups of one launch as 64-bit words (a tag in
// the high half, the value in the low half), written and polled with
// relaxed device-scope atomics, so no workgroup needs a device-scope fence,
// whose cache write-back and invalidation cost microseconds per workgroup:
// the router rows in launch 1, the parts of a down slab in launch 2. Launch
// 2 clears the router words, and each slab's last workgroup its slab's, so
// every call finds them at zero. A wait cannot deadlock: a waiting
// workgroup waits only on workgroups with lower indices (dispatched before
// it) that wait on nothing. A wait is still bounded: past the bound the
// workgroup sets a timeout word (sticky until the workspace is cleared) and
// the layer writes NaN to y.
#include <algorithm>
#include <atomic>

#include "decode.hpp"
#include "ffn_device.hpp"

namespace smoe {
namespace {

constexpr int kDW = 8;                  // waves per workgroup
constexpr int kDT = kDW * kWave;
constexpr int kSpinLimit = 1 << 22;     // polls before giving up (~0.2 s)
constexpr int kCtlTimeout = 0;          // ctl word: a wait ran out (sticky)
constexpr uint64_t kTag = 1ull << 32;   // high half of a published word

struct DArgs {
  FusedArgs f;
  const uint8_t *wg, *wu, *wd;          // routed INT4 codes, tiled
  const uint16_t *sg, *su, *sd;         // their scales, tiled
  const uint8_t *swg, *swu, *swd;       // shared FP16, tiled
  int E, H, I, Is, k;
  int nL, nS, nR;                       // router / shared / routed workgroups of launch 1
  int sp;                               // launch 2: parts of the shared expert's down K
  int* ctl;                             // [kCtlTimeout]
  uint64_t* lgw;                        // [E + 1]: router rows (row E: the raw gate dot)
  _Float16* h_r;                        // [k][I]
  _Float16* h_s;                        // [Is]
  uint64_t* partw;                      // [H/16][parts][16]: down sums of a slab's parts
  float* slot_out;
  float* shared_out;
  _Float16* y;
};

__device__ __forceinline__ int ld_agent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave: the published router rows [0, n) into lg (LDS), each lane
// polling its words until their tags are there; false when the wait ran
// out (the rows not there are NaN).
__device__ __forceinline__ bool gather_rows(const uint64_t* lgw, int n, float* lg, int lane) {
  constexpr int kPer = (kMaxE + 1 + kWave - 1) / kWave;
  bool ok = true;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = lane + i * kWave;
    if (r < n) {
      uint64_t w = ld_word(lgw + r);
      for (int m = 0; !(w & kTag) && m < kSpinLimit; ++m) {
        __builtin_amdgcn_s_sleep(1);
        w = ld_word(lgw + r);
      }
      ok = ok && (w & kTag) != 0;
      lg[r] = (w & kTag) ? bitcast<float>(static_cast<uint32_t>(w)) : __builtin_nanf("");
    }
  }
  return __all(ok);
}

// One router row for the one token, in the fixed fp32 order of
// smoe_route_topk: lane l sums the terms h = 64c + l in increasing c
// (product and sum each rounded), then the halving tree over the lanes,
// then the bias. Row E is the shared-gate vector (raw dot, no bias).
// Returns the row's value in lane 0.
__device__ __forceinline__ float router_row(const RouteArgs& a, int r, int lane) {
#pragma clang fp contract(off)
  const float* wr = r < a.E ? a.w + static_cast<size_t>(r) * a.H : a.gate_w;
  const int nc = a.H / kWave;
  constexpr int kChunk = 32;
  float p = 0.0f;
  for (int c0 = 0; c0 < nc; c0 += kChunk) {
    float wv[kChunk], xv[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int c = min(c0 + j, nc - 1);
      wv[j] = wr[c * kWave + lane];
      xv[j] = static_cast<float>(a.x[c * kWave + lane]);
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      if (c0 + j < nc) {
        const float prod = xv[j] * wv[j];
        p = p + prod;
      }
    }
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    const float o = __shfl_down(p, off, kWave);
    p = p + o;
  }
  if (r < a.E && a.bias != nullptr) p = p + a.bias[r];
  return p;  // (lane 0)
}

// sum_j b[j] * x[j] over 8 halves, in fp32
__device__ __forceinline__ float dot8(f16x8 b, f16x8 x, float c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 bb = {b[2 * i], b[2 * i + 1]};
    const f16x2 xx = {x[2 * i], x[2 * i + 1]};
    c = __builtin_amdgcn_fdot2(bb, xx, c, false);
  }
  return c;
}

// INT4 scales of one row of one block: NQ = 128 / G fp16 values
template <int G>
struct Scales {
  uint32_t v[G == 32 ? 2 : 1];
};
template <int G>
__device__ __forceinline__ Scales<G> load_scales(const uint16_t* p) {
  Scales<G> s;
  if constexpr (G == 128) {
    s.v[0] = gload<uint16_t>(p);
  } else if constexpr (G == 64) {
    s.v[0] = gload<uint32_t>(p);
  } else {
    const u32x2 v = gload<u32x2>(p);
    s.v[0] = v[0];
    s.v[1] = v[1];
  }
  return s;
}
template <int G>
__device__ __forceinline__ float scale_of(const Scales<G>& s, int gq) {
  const uint32_t w = s.v[G == 32 ? (gq >> 1) : 0];
  const uint16_t bits = static_cast<uint16_t>((gq & 1) ? (w >> 16) : w);
  return static_cast<float>(bitcast<_Float16>(bits));
}

// This lane's share of one INT4 block: lane (g, r) holds words
// int4_word(G, g, q) of row r; their halves meet the operand halves o[q].
template <int G>
__device__ __forceinline__ float dot_int4(u32x4 w, const Scales<G>& s, const f16x8* o,
                                          uint32_t lo, uint32_t hi, uint32_t magic) {
  constexpr int PER = G / 32;  // words per scale group
  float acc = 0.0f;
#pragma unroll
  for (int gq = 0; gq < 4 / PER; ++gq) {
    float d = 0.0f;
#pragma unroll
    for (int qq = 0; qq < PER; ++qq) {
      const int q = gq * PER + qq;
      d = dot8(dequant_word(w[q], lo, hi, magic), o[q], d);
    }
    acc += scale_of<G>(s, gq) * d;
  }
  return acc;
}

// the sum of a row's four lane groups, in every lane of the row
__device__ __forceinline__ float row_sum(float v) {
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}

struct UpSmem {
  float lg[kMaxE + 1];         // the router rows (workgroup 0 and the routed workgroups)
  uint64_t keys[kMaxE];        // the top-k's scratch
  int sel[kMaxK];
  int ids[kMaxK];              // workgroup 0: the top-k
  int pre[kMaxE];              // workgroup 0: the layer's counter row, read first
  int row[kMaxE];              // workgroup 0: a counter row being ranked
  float red[kDW][2][2][16];    // [wave][slab][gate, up][row]
  int bcast;
};

// The routing outputs of the one token, from its router rows in sm.lg: the
// same values as route_align_elb_block gives at T = 1, without its general
// machinery (k slots, each a distinct expert):
//   top-k and weights (the same wave routine), the shared gate's sigmoid;
//   counts[e] = 1 for a picked expert, offsets[e] = picked experts below e,
//   sorted_slots[offsets[ids[j]]] = j, active = the picked experts
//   ascending (then -1), n_active = k;
//   ELB: the layer's row gains one per picked expert; every layer's row is
//   ranked (count descending, ID ascending) into its top-M plan; with the
//   clear flag every row is then zeroed.
// Every output word is written once, after the loads; the barriers order
// LDS only.
__device__ void single_token_route(const FusedArgs& f, UpSmem& sm, int tid, int wave, int lane) {
  const RouteArgs& a = f.r;
  const int E = a.E, k = a.k;
  if (wave == 0) {
    int id;
    float w;
    wave_topk(sm.lg, E, k, a.flags, sm.keys, sm.sel, &id, &w);
    if (lane < k) {
      a.ids[lane] = id;
      a.wout[lane] = w;
      sm.ids[lane] = id;
    }
    if (a.gate != nullptr && a.gate_w != nullptr && lane == 0)
      a.gate[0] = 1.0f / (1.0f + expf(-sm.lg[E]));
    if (lane == 0) {
      f.offsets[E] = k;
      f.n_active[0] = k;
    }
  }
  block_sync_lds();
  if (tid < E) {
    int below = 0, picked = 0;
    for (int j = 0; j < k; ++j) {
      below += sm.ids[j] < tid ? 1 : 0;
      picked += sm.ids[j] == tid ? 1 : 0;
    }
    f.counts[tid] = picked;
    f.offsets[tid] = below;
    // active[i]: the picked expert with i picked experts below it
    int act = -1;
    for (int j = 0; j < k; ++j) {
      int r = 0;
      for (int i = 0; i < k; ++i) r += sm.ids[i] < sm.ids[j] ? 1 : 0;
      if (r == tid) act = sm.ids[j];
    }
    f.active[tid] = act;
  }
  if (tid < k) {
    int pos = 0;
    for (int i = 0; i < k; ++i) pos += sm.ids[i] < sm.ids[tid] ? 1 : 0;
    f.sorted_slots[pos] = tid;
  }
  if (f.elb_counts == nullptr) return;
  for (int l = 0; l < f.L; ++l) {
    int32_t* crow = f.elb_counts + static_cast<size_t>(l) * E;
    block_sync_lds();  // (the previous layer's ranking is done with sm.row)
    if (tid < E) {
      int v;
      if (l == f.layer) {
        int add = 0;
        for (int j = 0; j < k; ++j) add += sm.ids[j] == tid ? 1 : 0;
        v = sm.pre[tid] + add;
        if (add != 0) crow[tid] = v;
      } else {
        v = crow[tid];
      }
      sm.row[tid] = v;
    }
    block_sync_lds();
    if (f.M > 0 && tid < E) {
      const int c = sm.row[tid];
      int place = 0;
      for (int e2 = 0; e2 < E; ++e2) {
        const int c2 = sm.row[e2];
        place += (c2 > c || (c2 == c && e2 < tid)) ? 1 : 0;
      }
      if (place < f.M) {
        f.plan_ids[static_cast<size_t>(l) * f.M + place] = tid;
        if (f.plan_counts != nullptr) f.plan_counts[static_cast<size_t>(l) * f.M + place] = c;
      }
    }
    if (f.elb_clear && tid < E) crow[tid] = 0;
  }
}

template <int G>
__global__ __launch_bounds__(kDT) __attribute__((amdgpu_waves_per_eu(4))) void decode_up_kernel(
    DArgs a) {
  __shared__ UpSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int b = blockIdx.x;
  const _Float16* x = a.f.r.x;
  const bool gate_row = a.f.r.gate_w != nullptr;

  // ---- router rows, published; workgroup 0 then routes, aligns, counts
  if (b < a.nL) {
    // (workgroup 0 reads the layer's counter row before anything is stored)
    const int pre =
        b == 0 && a.f.elb_counts != nullptr && tid < a.E
            ? a.f.elb_counts[static_cast<size_t>(a.f.layer) * a.E + tid] : 0;
    const int r = b * kDW + wave;
    if (r < a.E || (r == a.E && gate_row)) {
      const float v = router_row(a.f.r, r, lane);
      if (lane == 0) st_word(a.lgw + r, kTag | bitcast<uint32_t>(v));
    }
    if (b != 0) return;
    if (tid < a.E) sm.pre[tid] = pre;
    const int nrow = a.E + (gate_row ? 1 : 0);
    if (wave == 0) {
      const bool ok = gather_rows(a.lgw, nrow, sm.lg, lane);
      if (lane == 0) sm.bcast = ok ? 1 : 0;
    }
    block_sync_lds();
    if (!sm.bcast) {
      if (tid == 0) st_agent(a.ctl + kCtlTimeout, 1);
      return;
    }
    if (tid < a.E) a.f.r.logits[tid] = sm.lg[tid];
    single_token_route(a.f, sm, tid, wave, lane);
    return;
  }

  uint32_t dq_lo = 0x000F000Fu, dq_hi = 0x00F000F0u, dq_magic = 0x64006400u;
  asm volatile("" : "+v"(dq_lo), "+v"(dq_hi), "+v"(dq_magic));  // keep the masks in VGPRs
  // gate and up sums of the workgroup's slabs (one shared slab, or two
  // slabs of one routed slot)
  float gs[2] = {0.0f, 0.0f}, us[2] = {0.0f, 0.0f};
  _Float16* out[2] = {nullptr, nullptr};

  if (b < a.nL + a.nS) {
    // ---- one 16-row slab of the shared gate and up (FP16, K = H)
    const int sl = b - a.nL;
    const int nblk = a.H / 32;
    const long long t0 = static_cast<long long>(sl) * nblk;
    constexpr int NB = 4;
    // The router rows go first: their few loads would otherwise queue behind
    // this stream and hold up every routed workgroup. (A timing gate only:
    // the shared expert needs no routing, and the wait is bounded.)
    if (tid == 0)
      for (int n = 0; n < kSpinLimit && !(ld_word(a.lgw + a.E - 1) & kTag); ++n)
        __builtin_amdgcn_s_sleep(2);
    block_sync_lds();
    for (int b0 = wave; b0 < nblk; b0 += NB * kDW) {
      u32x4 tg[NB], tu[NB];
      f16x8 xo[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int bk = min(b0 + i * kDW, nblk - 1);  // (past the end: loaded, not used)
        tg[i] = gload<u32x4>(a.swg + (t0 + bk) * 1024 + 16 * lane);
        tu[i] = gload<u32x4>(a.swu + (t0 + bk) * 1024 + 16 * lane);
        xo[i] = gload<f16x8>(x + bk * 32 + 8 * g);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (b0 + i * kDW < nblk) {
          gs[0] = dot8(bitcast<f16x8>(tg[i]), xo[i], gs[0]);
          us[0] = dot8(bitcast<f16x8>(tu[i]), xo[i], us[0]);
        }
      }
    }
    out[0] = a.h_s + sl * 16;
  } else {
    // ---- two 16-row slabs of slot j's expert, gate and up (INT4, K = H)
    const int slabs = a.I / 16;
    const int pairs = (slabs + 1) / 2;
    const int ri = b - a.nL - a.nS;
    const int j = ri / pairs, sl0 = 2 * (ri - j * pairs);
    const bool two = sl0 + 1 < slabs;
    const int nblk = a.H / 128;
    constexpr int NB = 2;
    // the activations of this wave's first blocks need no routing
    f16x8 xo[NB][4];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int bk = min(wave + i * kDW, nblk - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) xo[i][q] = gload<f16x8>(x + bk * 128 + 8 * int4_word(G, g, q));
    }
    // slot j's expert: the top-k of the published router rows
    if (wave == 0) {
      const bool ok = gather_rows(a.lgw, a.E, sm.lg, lane);
      int id = -1;
      float w = 0.0f;
      if (ok) {
        wave_topk(sm.lg, a.E, a.k, a.f.r.flags, sm.keys, sm.sel, &id, &w);
      } else if (lane == 0) {
        st_agent(a.ctl + kCtlTimeout, 1);
      }
      if (lane == j) sm.bcast = ok ? id : -1;
    }
    block_sync_lds();
    const int e = sm.bcast;
    if (e >= 0 && e < a.E) {
      constexpr int NQ = 128 / G;
      const long long t00 = (static_cast<long long>(e) * slabs + sl0) * nblk;
      for (int b0 = wave; b0 < nblk; b0 += NB * kDW) {
        u32x4 tg[2][NB], tu[2][NB];
        Scales<G> sg[2][NB], su[2][NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int bk = min(b0 + i * kDW, nblk - 1);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            // (the second slab of an odd count: the first loaded again, not used)
            const long long t = t00 + (two ? h : 0) * nblk + bk;
            tg[h][i] = gload<u32x4>(a.wg + t * 1024 + 16 * lane);
            tu[h][i] = gload<u32x4>(a.wu + t * 1024 + 16 * lane);
            sg[h][i] = load_scales<G>(a.sg + (t * 16 + r16) * NQ);
            su[h][i] = load_scales<G>(a.su + (t * 16 + r16) * NQ);
          }
          if (b0 != wave) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              xo[i][q] = gload<f16x8>(x + bk * 128 + 8 * int4_word(G, g, q));
          }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (b0 + i * kDW < nblk) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              gs[h] += dot_int4<G>(tg[h][i], sg[h][i], xo[i], dq_lo, dq_hi, dq_magic);
              us[h] += dot_int4<G>(tu[h][i], su[h][i], xo[i], dq_lo, dq_hi, dq_magic);
            }
          }
        }
      }
    }
    out[0] = a.h_r + static_cast<long long>(j) * a.I + sl0 * 16;
    if (two) out[1] = out[0] + 16;
  }

  // ---- rows: lane groups, then waves in order; h = SiLU(g) * u in fp16
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    gs[h] = row_sum(gs[h]);
    us[h] = row_sum(us[h]);
    if (lane < 16) {
      sm.red[wave][h][0][lane] = gs[h];
      sm.red[wave][h][1][lane] = us[h];
    }
  }
  block_sync_lds();
  _Float16* const o = wave == 0 ? out[0] : out[1];
  if (wave < 2 && lane < 16 && o != nullptr) {
    float gv = 0.0f, uv = 0.0f;
#pragma unroll
    for (int w = 0; w < kDW; ++w) {
      gv += sm.red[w][wave][0][lane];
      uv += sm.red[w][wave][1][lane];
    }
    const float hv = gv / (1.0f + __expf(-gv)) * uv;
    o[lane] = static_cast<_Float16>(hv);
  }
}

constexpr int kDW2 = 8;                 // waves per workgroup of launch 2
constexpr int kDT2 = kDW2 * kWave;
constexpr int kMaxSharedParts = 8;      // parts of the shared expert's down K

// Launch 2: one workgroup per (16-row slab of the output, part): a routed
// slot's down rows (I / 128 blocks), or a share of the shared expert's K.
// The slab's last part gathers the others. Launch 2 also clears the router
// words for the next call.
// (four workgroups per CU: about every workgroup of the launch is resident)
template <int G>
__global__ __launch_bounds__(kDT2) __attribute__((amdgpu_waves_per_eu(8))) void decode_down_kernel(
    DArgs a) {
  __shared__ float red[kDW2][16];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  if (blockIdx.x == 0)
    for (int i = tid; i <= a.E; i += kDT2) st_word(a.lgw + i, 0);
  const int np = a.k + a.sp;
  const int item = blockIdx.x;
  const int sl = item / np, part = item - sl * np;
  uint32_t dq_lo = 0x000F000Fu, dq_hi = 0x00F000F0u, dq_magic = 0x64006400u;
  asm volatile("" : "+v"(dq_lo), "+v"(dq_hi), "+v"(dq_magic));
  float acc = 0.0f;
  if (part < a.k) {
    // ---- slot `part`: rows of its expert's down matrix (INT4, K = I)
    const int e = a.f.r.ids[part];
    if (e >= 0 && e < a.E) {
      const int nblk = a.I / 128;
      const long long t0 = (static_cast<long long>(e) * (a.H / 16) + sl) * nblk;
      const _Float16* h = a.h_r + static_cast<long long>(part) * a.I;
      constexpr int NQ = 128 / G;
      constexpr int NB = 2;
      for (int b0 = wave; b0 < nblk; b0 += NB * kDW2) {
        u32x4 tw[NB];
        Scales<G> sw[NB];
        f16x8 ho[NB][4];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int bk = min(b0 + i * kDW2, nblk - 1);  // (past the end: loaded, not used)
          const long long t = t0 + bk;
          tw[i] = gload<u32x4>(a.wd + t * 1024 + 16 * lane);
          sw[i] = load_scales<G>(a.sd + (t * 16 + r16) * NQ);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            ho[i][q] = gload<f16x8>(h + bk * 128 + 8 * int4_word(G, g, q));
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
          if (b0 + i * kDW2 < nblk)
            acc += dot_int4<G>(tw[i], sw[i], ho[i], dq_lo, dq_hi, dq_magic);
      }
    }
  } else {
    // ---- one part of the shared down matrix's K (FP16, K = Is)
    const int q = part - a.k;
    const int nblk = a.Is / 32;
    const int lo = q * nblk / a.sp, hi = (q + 1) * nblk / a.sp;
    const long long t0 = static_cast<long long>(sl) * nblk;
    constexpr int NB = 6;
    for (int b0 = lo + wave; b0 < hi; b0 += NB * kDW2) {
      u32x4 tw[NB];
      f16x8 ho[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int bk = min(b0 + i * kDW2, hi - 1);
        tw[i] = gload<u32x4>(a.swd + (t0 + bk) * 1024 + 16 * lane);
        ho[i] = gload<f16x8>(a.h_s + bk * 32 + 8 * g);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (b0 + i * kDW2 < hi) acc = dot8(bitcast<f16x8>(tw[i]), ho[i], acc);
    }
  }

  // ---- this part's 16 rows; the slab's last part combines them all
  acc = row_sum(acc);
  if (lane < 16) red[wave][lane] = acc;
  block_sync_lds();
  if (wave != 0 || lane >= 16) return;
  float v = 0.0f;
#pragma unroll
  for (int w = 0; w < kDW2; ++w) v += red[w][lane];
  uint64_t* ws = a.partw + static_cast<long long>(sl) * np * 16 + lane;
  if (part != np - 1) {
    st_word(ws + part * 16, kTag | bitcast<uint32_t>(v));
    return;
  }
  // the other parts' words, all polled in each round, then back to zero
  constexpr int kMaxParts = kMaxK + kMaxSharedParts;
  float pv[kMaxParts];
  bool have[kMaxParts];
#pragma unroll
  for (int p = 0; p < kMaxParts; ++p) {
    pv[p] = v;
    have[p] = p >= np - 1;
  }
  bool ok = false;
  for (int n = 0; n < kSpinLimit && !ok; ++n) {
    ok = true;
#pragma unroll
    for (int p = 0; p < kMaxParts; ++p) {
      if (!have[p]) {
        const uint64_t w = ld_word(ws + p * 16);
        have[p] = (w & kTag) != 0;
        pv[p] = bitcast<float>(static_cast<uint32_t>(w));
        ok = ok && have[p];
      }
    }
    if (!ok) __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int p = 0; p < kMaxParts; ++p)
    if (p < np - 1) st_word(ws + p * 16, 0);
  const int n = sl * 16 + lane;
  float yv = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < a.k) {
      a.slot_out[static_cast<long long>(j) * a.H + n] = pv[j];
      yv += a.f.r.wout[j] * pv[j];
    }
  }
  if (a.Is > 0) {
    float sh = 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxSharedParts; ++q)
      if (q < a.sp) sh += pv[a.k + q];
    a.shared_out[n] = sh;
    const float gate = a.f.r.gate != nullptr && a.f.r.gate_w != nullptr ? a.f.r.gate[0] : 1.0f;
    yv += gate * sh;
  }
  if (!ok) st_agent(a.ctl + kCtlTimeout, 1);
  if (!ok || ld_agent(a.ctl + kCtlTimeout) != 0) yv = __builtin_nanf("");
  a.y[n] = static_cast<_Float16>(yv);
}

size_t round256(long long v) { return static_cast<size_t>((v + 255) / 256 * 256); }

template <int G>
smoe_status launch_decode(const DArgs& a, hipStream_t st, const char* who) {
  const int grid1 = a.nL + a.nS + a.nR;
  hipLaunchKernelGGL(decode_up_kernel<G>, dim3(grid1), dim3(kDT), 0, st, a);
  smoe_status s = check_launch(who);
  if (s != SMOE_OK) return s;
  hipLaunchKernelGGL(decode_down_kernel<G>, dim3(a.H / 16 * (a.k + a.sp)), dim3(kDT2), 0, st, a);
  return check_launch(who);
}

}  // namespace

// parts of the shared expert's down K: about four routed slots' blocks each
int shared_parts(long long I, long long Is) {
  if (Is <= 0) return 0;
  const long long per = 4 * (I / 128), nblk = Is / 32;
  return static_cast<int>(std::min<long long>(kMaxSharedParts, std::max(1ll, (nblk + per - 1) / per)));
}

size_t decode_region_bytes(long long k, long long H, long long I, long long Is) {
  const long long np = k + shared_parts(I, Is);
  return 256 + round256((kMaxE + 1) * 8) + round256(k * I * 2) + round256(Is * 2) +
         round256(H / 16 * np * 16 * 8);
}

bool decode_applicable(int T, int k, int E, int H, int I, int Is, int G) {
  return T == 1 && k >= 1 && k <= kMaxK && E >= k && E <= kMaxE && H % 128 == 0 &&
         H <= 8192 && I % 128 == 0 && Is % 128 == 0 && (G == 32 || G == 64 || G == 128);
}

smoe_status decode_layer(const DecodeCall& c, hipStream_t st, const char* who) {
  DArgs a{};
  a.f = c.f;
  a.wg = static_cast<const uint8_t*>(c.wg);
  a.wu = static_cast<const uint8_t*>(c.wu);
  a.wd = static_cast<const uint8_t*>(c.wd);
  a.sg = static_cast<const uint16_t*>(c.sg);
  a.su = static_cast<const uint16_t*>(c.su);
  a.sd = static_cast<const uint16_t*>(c.sd);
  a.swg = static_cast<const uint8_t*>(c.swg);
  a.swu = static_cast<const uint8_t*>(c.swu);
  a.swd = static_cast<const uint8_t*>(c.swd);
  a.E = c.f.r.E;
  a.H = c.f.r.H;
  a.I = c.I;
  a.Is = c.Is;
  a.k = c.f.r.k;
  const bool gate_row = c.f.r.gate_w != nullptr;
  a.nL = (a.E + (gate_row ? 1 : 0) + kDW - 1) / kDW;
  a.nS = a.Is / 16;
  a.nR = a.k * ((a.I / 16 + 1) / 2);
  a.sp = shared_parts(a.I, a.Is);
  uint8_t* p = static_cast<uint8_t*>(c.region);
  a.ctl = reinterpret_cast<int*>(p);
  p += 256;
  a.lgw = reinterpret_cast<uint64_t*>(p);
  p += round256((kMaxE + 1) * 8);
  a.h_r = reinterpret_cast<_Float16*>(p);
  p += round256(static_cast<long long>(a.k) * a.I * 2);  // (k I 2 is a 256 multiple)
  a.h_s = reinterpret_cast<_Float16*>(p);
  p += round256(static_cast<long long>(a.Is) * 2);
  a.partw = reinterpret_cast<uint64_t*>(p);
  a.slot_out = c.slot_out;
  a.shared_out = c.shared_out;
  a.y = static_cast<_Float16*>(c.y);
  switch (c.G) {
    case 32: return launch_decode<32>(a, st, who);
    case 64: return launch_decode<64>(a, st, who);
    default: return launch_decode<128>(a, st, who);
  }
}

}  // namespace smoe
