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
//   stage 1  h[p] = fp16( SiLU(x_t . Wg^T) * (x_t . Wu^T) )   p = sorted slot position
//   stage 2  slot_out[s] = h[p] . Wd^T                        s = sorted_slots[p]
// Work item = one wave = (expert, chunk of up to 16*NC of its slots, 16-row
// tile of gate and up  |  two 16-row tiles of down). The wave streams its
// weight rows once over the whole reduction length K and applies them to
// every slot of the chunk, so each expert's weights leave HBM once per chunk.
//
// MFMA mapping (v_mfma_f32_16x16x32_f16, wave64): A = activations (16 slot
// rows x 32 k), B = weights (32 k x 16 weight rows), D[slot][row]. Lane l
// feeds slot / weight row l % 16 and the k-set of lane group l / 16, and
// holds D for slots 4*(l/16) + 0..3 of weight row l % 16 -- so every
// accumulator of a lane belongs to one weight row, and the INT4 group scale
// of that row is applied once per group in FP32 after the group's MFMAs.
//
// INT4 dequantisation without lookup tables: a packed word w holds 8 codes;
// (w >> 4i) & 0x000F000F | 0x64006400 read as two fp16 values is
// (1024 + c_i, 1024 + c_{i+4}); subtracting 1032 gives c - 8 exactly. The
// eight values come out in k order 0,4,1,5,2,6,3,7, so the activation
// operand is permuted the same way (x when it is loaded; h by storing it
// permuted within each group of 8 when stage 1 writes it).
//
// Per 128-k block a lane of group g covers the words of its group:
//   G = 128: words 4g .. 4g+3 of the block (one 16-byte load);
//   G =  64: words 2g, 2g+1 of each 64-k half (two 8-byte loads);
//   G =  32: word g of each 32-k quarter (four 4-byte loads);
// so each MFMA's 32 k lie in one quantisation group.
//
// Loads are software-pipelined DEPTH blocks ahead; weights, scales and the
// activation operand of a block are issued together so the in-order vector
// memory counter never makes one block wait on a later block's loads.
//
// Work mapping: grid = 8 * ceil(max_chunks / 8) * n_tiles one-wave
// workgroups; workgroup b runs on XCD b % 8 and takes chunk
// 8 * ((b / 8) / n_tiles) + b % 8, tile (b / 8) % n_tiles, so all tiles of a
// chunk share one XCD's L2 (its activations are fetched once per XCD), and
// the chunks are spread evenly over the XCDs. A chunk index is turned into
// (expert, slot range) on the device from expert_offsets with a wave prefix
// sum, so nothing is read back to the host.
#include <algorithm>

#include "smoe_internal.hpp"

namespace smoe {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { kInt4 = 0, kFp16 = 1 };
constexpr int kKB = 128;  // k per block

struct FfnArgs {
  const uint16_t* act;          // stage 1: x [T][K]; stage 2: h [S][K] (fp16 bits)
  const int32_t* sorted_slots;  // [S]
  const int32_t* offsets;       // [E+1]
  const uint8_t* w0;            // stage 1: gate; stage 2: down
  const uint8_t* w1;            // stage 1: up
  const uint16_t* s0;           // INT4 scales of w0 / w1 (fp16 bits)
  const uint16_t* s1;
  uint16_t* h;                  // stage 1 output [S][N]
  float* out;                   // stage 2 output [S][N], row = slot
  size_t w_estride;             // bytes per expert
  size_t w_rstride;             // bytes per weight row
  size_t s_estride;             // scale elements per expert
  int s_rstride;                // scale elements per row
  int E, k, K, N;
  int n_tiles;
  int max_chunks;
};

template <typename T, typename U>
__device__ __forceinline__ T bitcast(U u) {
  static_assert(sizeof(T) == sizeof(U), "size");
  T t;
  __builtin_memcpy(&t, &u, sizeof(T));
  return t;
}

// (expert, slot range) of chunk `chunk`, chunks of MT slots numbered expert
// by expert in ID order. Returns false past the last chunk.
template <int MT>
__device__ __forceinline__ bool locate_chunk(const int32_t* __restrict__ offsets, int E,
                                             int chunk, int& e_out, int& seg0, int& seg1) {
  const int lane = lane_id();
  int o[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) o[i] = offsets[min(4 * lane + i, E)];
  int nch[4], tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    nch[i] = (o[i + 1] - o[i] + MT - 1) / MT;
    tot += nch[i];
  }
  const int incl = wave_inclusive_scan(tot);
  const int start = incl - tot;
  const bool mine = chunk >= start && chunk < incl;
  const uint64_t m = __ballot(mine);
  if (m == 0ull) return false;
  int e_l = 0, s0_l = 0, s1_l = 0, c0 = start;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (chunk >= c0 && chunk < c0 + nch[i]) {
      e_l = 4 * lane + i;
      s0_l = o[i] + (chunk - c0) * MT;
      s1_l = min(s0_l + MT, o[i + 1]);
    }
    c0 += nch[i];
  }
  const int src = __ffsll(static_cast<long long>(m)) - 1;
  e_out = __shfl(e_l, src, kWave);
  seg0 = __shfl(s0_l, src, kWave);
  seg1 = __shfl(s1_l, src, kWave);
  return true;
}

// Eight INT4 codes of one word -> (c - 8) as fp16, in k order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ f16x8 dequant_word(uint32_t w) {
  const uint32_t lo = 0x000F000Fu, magic = 0x64006400u;
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

// Physical column of logical column n in an h row that feeds INT4 weights.
__device__ __forceinline__ int h_perm_col(int n) {
  const int q = n & 7;
  return (n & ~7) | (((q & 3) << 1) | (q >> 2));
}

// Word index (within a 128-k block) that MFMA slot c of lane group g uses.
template <int G>
__device__ __forceinline__ int int4_word(int g, int c) {
  constexpr int per = G / 32;  // MFMAs per group
  return (c / per) * (G / 8) + g * per + (c % per);
}

template <int WK, int NC>
struct BlockRegs {
  u32x4 w[2][WK == kInt4 ? 1 : 4];
  uint32_t s[2][2];
  u32x4 x[NC][4];
};

template <int WK, int G, int NC, int STAGE, int DEPTH>
__global__ __launch_bounds__(64) void ffn_kernel(FfnArgs a) {
  constexpr int MT = 16 * NC;
  constexpr int NQ = kKB / G;  // quantisation groups per block (INT4)
  constexpr bool PERM_LOAD = (WK == kInt4) && (STAGE == 1);
  const int lane = threadIdx.x;
  const int g = lane >> 4;
  const int r16 = lane & 15;

  const int b = blockIdx.x;
  const int j = b >> 3;
  const int chunk = (j / a.n_tiles) * 8 + (b & 7);
  const int tile = j % a.n_tiles;
  if (chunk >= a.max_chunks) return;
  int e, seg0, seg1;
  if (!locate_chunk<MT>(a.offsets, a.E, chunk, e, seg0, seg1)) return;

  // weight rows of this lane for the two matrices
  const uint8_t* wrow[2];
  const uint16_t* srow[2];
  int nrow[2];
  if (STAGE == 1) {
    nrow[0] = nrow[1] = tile * 16 + r16;
    wrow[0] = a.w0 + e * a.w_estride + nrow[0] * a.w_rstride;
    wrow[1] = a.w1 + e * a.w_estride + nrow[1] * a.w_rstride;
    if (WK == kInt4) {
      srow[0] = a.s0 + e * a.s_estride + static_cast<size_t>(nrow[0]) * a.s_rstride;
      srow[1] = a.s1 + e * a.s_estride + static_cast<size_t>(nrow[1]) * a.s_rstride;
    }
  } else {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      nrow[m] = tile * 32 + m * 16 + r16;
      wrow[m] = a.w0 + e * a.w_estride + nrow[m] * a.w_rstride;
      if (WK == kInt4)
        srow[m] = a.s0 + e * a.s_estride + static_cast<size_t>(nrow[m]) * a.s_rstride;
    }
  }

  // activation row of this lane (A operand) for each chunk of 16 slots
  const uint16_t* arow[NC];
  bool avalid[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int p = seg0 + 16 * c + r16;
    avalid[c] = p < seg1;
    arow[c] = a.act;
    if (avalid[c]) {
      if (STAGE == 1) {
        const int slot = a.sorted_slots[p];
        arow[c] = a.act + static_cast<size_t>(slot / a.k) * a.K;
      } else {
        arow[c] = a.act + static_cast<size_t>(p) * a.K;
      }
    }
  }

  auto load_block = [&](BlockRegs<WK, NC>& r, int blk) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (WK == kInt4) {
        const uint8_t* base = wrow[m] + blk * (kKB / 2);
        if (G == 128) {
          r.w[m][0] = *reinterpret_cast<const u32x4*>(base + 16 * g);
        } else if (G == 64) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(base + 8 * g);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(base + 32 + 8 * g);
          r.w[m][0] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            r.w[m][0][q] = *reinterpret_cast<const uint32_t*>(base + 16 * q + 4 * g);
        }
        const uint16_t* sp = srow[m] + blk * NQ;
        if (NQ == 1) {
          r.s[m][0] = *sp;
        } else if (NQ == 2) {
          r.s[m][0] = *reinterpret_cast<const uint32_t*>(sp);
        } else {
          const u32x2 v = *reinterpret_cast<const u32x2*>(sp);
          r.s[m][0] = v[0];
          r.s[m][1] = v[1];
        }
      } else {
        const u32x4* base = reinterpret_cast<const u32x4*>(wrow[m] + blk * (kKB * 2) + 64 * g);
#pragma unroll
        for (int c = 0; c < 4; ++c) r.w[m][c] = base[c];
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k0 = blk * kKB + (WK == kInt4 ? 8 * int4_word<G>(g, q) : 32 * g + 8 * q);
        r.x[c][q] = avalid[c] ? *reinterpret_cast<const u32x4*>(arow[c] + k0) : u32x4{0, 0, 0, 0};
      }
    }
  };

  f32x4 acc[2][NC];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[m][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute_block = [&](const BlockRegs<WK, NC>& r) {
    f16x8 A[NC][4];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        A[c][q] = bitcast<f16x8>(PERM_LOAD ? permute_k8(r.x[c][q]) : r.x[c][q]);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (WK == kInt4) {
        f16x8 B[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) B[q] = dequant_word(r.w[m][0][q]);
#pragma unroll
        for (int grp = 0; grp < NQ; ++grp) {
          constexpr int per = G / 32;
          const uint32_t sbits = (NQ == 4) ? (r.s[m][grp >> 1] >> (16 * (grp & 1)))
                                           : (r.s[m][0] >> (16 * grp));
          const float sc =
              static_cast<float>(bitcast<_Float16>(static_cast<uint16_t>(sbits & 0xFFFFu)));
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int q = 0; q < per; ++q)
              t = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[c][grp * per + q], B[grp * per + q], t,
                                                         0, 0, 0);
            acc[m][c] += sc * t;
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f16x8 B = bitcast<f16x8>(r.w[m][q]);
#pragma unroll
          for (int c = 0; c < NC; ++c)
            acc[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[c][q], B, acc[m][c], 0, 0, 0);
        }
      }
    }
  };

  const int nblk = a.K / kKB;
  BlockRegs<WK, NC> ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (d < nblk) load_block(ring[d], d);
  for (int blk0 = 0; blk0 < nblk; blk0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int blk = blk0 + d;
      if (blk < nblk) {
        compute_block(ring[d]);
        if (blk + DEPTH < nblk) load_block(ring[d], blk + DEPTH);
      }
    }
  }

  // epilogue: lane holds D[slot 4g + i][row r16] of each chunk and matrix
  if (STAGE == 1) {
    const int col = WK == kInt4 ? h_perm_col(nrow[0]) : nrow[0];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = seg0 + 16 * c + 4 * g + i;
        if (p < seg1) {
          const float gv = acc[0][c][i], uv = acc[1][c][i];
          const float hv = gv / (1.0f + __expf(-gv)) * uv;
          a.h[static_cast<size_t>(p) * a.N + col] = bitcast<uint16_t>(static_cast<_Float16>(hv));
        }
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = seg0 + 16 * c + 4 * g + i;
        if (p < seg1) {
          const int slot = a.sorted_slots[p];
          float* dst = a.out + static_cast<size_t>(slot) * a.N;
          dst[nrow[0]] = acc[0][c][i];
          dst[nrow[1]] = acc[1][c][i];
        }
      }
    }
  }
}

// Slots per chunk: enough 16-slot MFMA column groups that the expected
// number of slots per active expert fits one chunk (up to 64).
int choose_nc(int S, int E) {
  const int active = std::min(E, S);
  const int mean = active > 0 ? (S + active - 1) / active : 1;
  return mean <= 16 ? 1 : (mean <= 32 ? 2 : 4);
}

template <int WK, int G, int NC>
smoe_status launch_ffn(FfnArgs a1, FfnArgs a2, int grid_slots, hipStream_t st) {
  constexpr int DEPTH = WK == kInt4 ? 3 : 2;
  const int g1 = 8 * grid_slots * a1.n_tiles;
  const int g2 = 8 * grid_slots * a2.n_tiles;
  hipLaunchKernelGGL((ffn_kernel<WK, G, NC, 1, DEPTH>), dim3(g1), dim3(64), 0, st, a1);
  smoe_status s = check_launch("expert_ffn stage 1");
  if (s != SMOE_OK) return s;
  hipLaunchKernelGGL((ffn_kernel<WK, G, NC, 2, DEPTH>), dim3(g2), dim3(64), 0, st, a2);
  return check_launch("expert_ffn stage 2");
}

template <int WK, int G>
smoe_status launch_nc(int nc, FfnArgs a1, FfnArgs a2, int grid_slots, hipStream_t st) {
  switch (nc) {
    case 1: return launch_ffn<WK, G, 1>(a1, a2, grid_slots, st);
    case 2: return launch_ffn<WK, G, 2>(a1, a2, grid_slots, st);
    default: return launch_ffn<WK, G, 4>(a1, a2, grid_slots, st);
  }
}

size_t workspace_bytes(long long S, long long I) {
  const size_t h = static_cast<size_t>(S) * static_cast<size_t>(I) * 2;
  return (h + 255) & ~static_cast<size_t>(255);
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
  SMOE_REQUIRE(static_cast<long long>(T) * k < (1ll << 24), SMOE_EUNSUPPORTED,
               "%s: T*k must be below 2^24", who);
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(x && sorted_slots && offsets && workspace && slot_out, SMOE_EINVAL,
               "%s: null pointer", who);
  SMOE_REQUIRE(ws_bytes >= workspace_bytes(static_cast<long long>(T) * k, I), SMOE_EINVAL,
               "%s: workspace of %zu bytes is below the %zu needed", who, ws_bytes,
               workspace_bytes(static_cast<long long>(T) * k, I));
  SMOE_REQUIRE(aligned16(x) && aligned16(workspace) && aligned16(slot_out), SMOE_EINVAL,
               "%s: x, workspace and slot_out must be 16-byte aligned", who);
  return SMOE_OK;
}

}  // namespace
}  // namespace smoe

using namespace smoe;

extern "C" size_t smoe_ffn_workspace_bytes(int T, int k, int E, int H, int I) {
  if (T < 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0) return 0;
  return workspace_bytes(static_cast<long long>(T) * k, I);
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
  smoe_status st = check_common("w4a16_expert_ffn", x, T, k, E, H, I, sorted_slots,
                                expert_offsets, workspace, workspace_bytes_, slot_out);
  if (st != SMOE_OK) return st;
  SMOE_REQUIRE(group_size == 32 || group_size == 64 || group_size == 128, SMOE_EUNSUPPORTED,
               "w4a16_expert_ffn: group size must be 32, 64 or 128 (got %d)", group_size);
  if (T == 0) return SMOE_OK;
  SMOE_REQUIRE(wg_q && wg_s && wu_q && wu_s && wd_q && wd_s, SMOE_EINVAL,
               "w4a16_expert_ffn: null weight pointer");
  SMOE_REQUIRE(aligned16(wg_q) && aligned16(wu_q) && aligned16(wd_q), SMOE_EINVAL,
               "w4a16_expert_ffn: packed weights must be 16-byte aligned");
  SMOE_REQUIRE(((reinterpret_cast<uintptr_t>(wg_s) | reinterpret_cast<uintptr_t>(wu_s) |
                 reinterpret_cast<uintptr_t>(wd_s)) & 7u) == 0,
               SMOE_EINVAL, "w4a16_expert_ffn: scales must be 8-byte aligned");
  const int S = T * k;
  const int nc = choose_nc(S, E);
  const int mt = 16 * nc;
  const int max_chunks = std::min(E, S) + S / mt;
  const int grid_slots = (max_chunks + 7) / 8;

  FfnArgs a1{};
  a1.act = static_cast<const uint16_t*>(x);
  a1.sorted_slots = sorted_slots;
  a1.offsets = expert_offsets;
  a1.w0 = reinterpret_cast<const uint8_t*>(wg_q);
  a1.w1 = reinterpret_cast<const uint8_t*>(wu_q);
  a1.s0 = static_cast<const uint16_t*>(wg_s);
  a1.s1 = static_cast<const uint16_t*>(wu_s);
  a1.h = static_cast<uint16_t*>(workspace);
  a1.w_rstride = static_cast<size_t>(H) / 2;
  a1.w_estride = a1.w_rstride * I;
  a1.s_rstride = H / group_size;
  a1.s_estride = static_cast<size_t>(a1.s_rstride) * I;
  a1.E = E; a1.k = k; a1.K = H; a1.N = I;
  a1.n_tiles = I / 16;
  a1.max_chunks = max_chunks;

  FfnArgs a2 = a1;
  a2.act = static_cast<const uint16_t*>(workspace);
  a2.w0 = reinterpret_cast<const uint8_t*>(wd_q);
  a2.w1 = nullptr;
  a2.s0 = static_cast<const uint16_t*>(wd_s);
  a2.s1 = nullptr;
  a2.h = nullptr;
  a2.out = slot_out;
  a2.w_rstride = static_cast<size_t>(I) / 2;
  a2.w_estride = a2.w_rstride * H;
  a2.s_rstride = I / group_size;
  a2.s_estride = static_cast<size_t>(a2.s_rstride) * H;
  a2.K = I; a2.N = H;
  a2.n_tiles = H / 32;

  hipStream_t s = as_stream(stream);
  switch (group_size) {
    case 32: return launch_nc<kInt4, 32>(nc, a1, a2, grid_slots, s);
    case 64: return launch_nc<kInt4, 64>(nc, a1, a2, grid_slots, s);
    default: return launch_nc<kInt4, 128>(nc, a1, a2, grid_slots, s);
  }
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
  const int S = T * k;
  const int nc = choose_nc(S, E);
  const int mt = 16 * nc;
  const int max_chunks = std::min(E, S) + S / mt;
  const int grid_slots = (max_chunks + 7) / 8;

  FfnArgs a1{};
  a1.act = static_cast<const uint16_t*>(x);
  a1.sorted_slots = sorted_slots;
  a1.offsets = expert_offsets;
  a1.w0 = static_cast<const uint8_t*>(wg);
  a1.w1 = static_cast<const uint8_t*>(wu);
  a1.h = static_cast<uint16_t*>(workspace);
  a1.w_rstride = static_cast<size_t>(H) * 2;
  a1.w_estride = a1.w_rstride * I;
  a1.E = E; a1.k = k; a1.K = H; a1.N = I;
  a1.n_tiles = I / 16;
  a1.max_chunks = max_chunks;

  FfnArgs a2 = a1;
  a2.act = static_cast<const uint16_t*>(workspace);
  a2.w0 = static_cast<const uint8_t*>(wd);
  a2.w1 = nullptr;
  a2.h = nullptr;
  a2.out = slot_out;
  a2.w_rstride = static_cast<size_t>(I) * 2;
  a2.w_estride = a2.w_rstride * H;
  a2.K = I; a2.N = H;
  a2.n_tiles = H / 32;
  return launch_nc<kFp16, 128>(nc, a1, a2, grid_slots, as_stream(stream));
}
