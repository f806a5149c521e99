// smoe_tile_weights: rewrites expert weights from the row-major layout into
// the 16-row tiled layout that the expert FFN streams in one piece per load.
//
// The tiled layout holds the same bytes as the row-major one, in another
// order (the values, codes and scales are unchanged). For each expert e,
// each slice of 16 rows (sl = row / 16) and each block of k (64 bytes of one
// row: 128 INT4 codes or 32 FP16 values), one kilobyte:
//   byte 16 * (16 g + r) + 4 q .. +3 = word W(g, q) of row 16 sl + r, block b
// with W(g, q) = 4 g + q for FP16 and INT4 G = 128, and the FFN's step-order
// word of lane group g for INT4 G = 64 and 32 (int4_word). Slices follow
// each other in row order, blocks in k order within a slice. Each INT4 word
// has its nibbles unzipped: the codes of k = 8w + 2p sit in nibble positions
// p = 0..3 and those of k = 8w + 2p + 1 in positions 4 + p, so that the
// FFN's dequantisation, which pairs positions (0, 4), (1, 5), (2, 6), (3, 7),
// yields the eight values in natural k order. INT4 scales:
// for each (e, sl, b), 16 runs of NQ = 128 / G values, run r holding the
// scales of row 16 sl + r that fall in block b.
//
// One thread per 16 output bytes (and per row and block of scales); the
// reads are 4-byte, the writes 16-byte and coalesced. Weights are tiled
// once when they are loaded, so this is not on the hot path.
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kTileThreads = 256;

// Natural nibble order (k = 8w + j in nibble j) -> even k in nibbles 0..3,
// odd k in nibbles 4..7.
__device__ __forceinline__ uint32_t unzip_nibbles(uint32_t w) {
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pos = (j & 1) ? 4 + (j >> 1) : (j >> 1);
    r |= ((w >> (4 * j)) & 0xFu) << (4 * pos);
  }
  return r;
}

template <int G, bool UNZIP>
__global__ __launch_bounds__(kTileThreads) void tile_codes_kernel(
    const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, long long n_chunks, int nblk) {
  const long long i = static_cast<long long>(blockIdx.x) * kTileThreads + threadIdx.x;
  if (i >= n_chunks) return;
  // i = ((e * N/16 + sl) * nblk + b) * 64 + lane; rows are contiguous across
  // (e, sl), so the row is (i / 64 / nblk) * 16 + lane % 16
  const int lane = static_cast<int>(i & 63);
  const long long tb = i >> 6;
  const long long slice = tb / nblk;
  const int b = static_cast<int>(tb - slice * nblk);
  const long long row = slice * 16 + (lane & 15);
  const int g = lane >> 4;
  const uint32_t* s = src + (row * nblk + b) * 16;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q] = s[int4_word(G, g, q)];
    if (UNZIP) w[q] = unzip_nibbles(w[q]);
  }
  reinterpret_cast<uint4*>(dst)[i] = uint4{w[0], w[1], w[2], w[3]};
}

template <int NQ>
__global__ __launch_bounds__(kTileThreads) void tile_scales_kernel(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, long long n_runs, int nblk) {
  const long long i = static_cast<long long>(blockIdx.x) * kTileThreads + threadIdx.x;
  if (i >= n_runs) return;
  // i = ((e * N/16 + sl) * nblk + b) * 16 + r
  const int r = static_cast<int>(i & 15);
  const long long tb = i >> 4;
  const long long slice = tb / nblk;
  const int b = static_cast<int>(tb - slice * nblk);
  const long long row = slice * 16 + r;
#pragma unroll
  for (int j = 0; j < NQ; ++j) dst[i * NQ + j] = src[(row * nblk + b) * NQ + j];
}

int grid_of(long long n) { return static_cast<int>((n + kTileThreads - 1) / kTileThreads); }

}  // namespace
}  // namespace smoe

using namespace smoe;

extern "C" smoe_status smoe_tile_weights(const void* w, const void* scales, int E, int N, int K,
                                         int group_size, void* w_tiled, void* scales_tiled,
                                         void* stream) {
  clear_error();
  const char* who = "tile_weights";
  SMOE_REQUIRE(E >= 0 && N >= 0 && K >= 0, SMOE_EINVAL,
               "%s: need E, N, K >= 0 (E=%d N=%d K=%d)", who, E, N, K);
  SMOE_REQUIRE(group_size == 0 || group_size == 32 || group_size == 64 || group_size == 128,
               SMOE_EUNSUPPORTED, "%s: group size must be 0 (FP16), 32, 64 or 128 (got %d)", who,
               group_size);
  SMOE_REQUIRE(N % 16 == 0 && K % 128 == 0, SMOE_EUNSUPPORTED,
               "%s: need N a multiple of 16 and K of 128 (N=%d K=%d)", who, N, K);
  const bool int4 = group_size != 0;
  const long long rows = static_cast<long long>(E) * N;
  if (rows == 0 || K == 0) return SMOE_OK;
  SMOE_REQUIRE(w && w_tiled, SMOE_EINVAL, "%s: null weight pointer", who);
  SMOE_REQUIRE(!int4 || (scales && scales_tiled), SMOE_EINVAL, "%s: null scale pointer", who);
  SMOE_REQUIRE(aligned16(w) && aligned16(w_tiled) &&
                   (!int4 || (aligned16(scales) && aligned16(scales_tiled))),
               SMOE_EINVAL, "%s: buffers must be 16-byte aligned", who);
  const int row_bytes = int4 ? K / 2 : 2 * K;
  const int nblk = row_bytes / 64;
  const long long bytes = rows * row_bytes;
  const char* wb = static_cast<const char*>(w);
  const char* db = static_cast<const char*>(w_tiled);
  SMOE_REQUIRE(db + bytes <= wb || wb + bytes <= db, SMOE_EINVAL,
               "%s: w_tiled must not overlap w", who);
  const long long n_runs = rows * nblk;
  const long long sbytes = int4 ? rows * (K / group_size) * 2 : 0;
  const char* sb = static_cast<const char*>(scales);
  const char* tb = static_cast<const char*>(scales_tiled);
  SMOE_REQUIRE(!int4 || tb + sbytes <= sb || sb + sbytes <= tb, SMOE_EINVAL,
               "%s: scales_tiled must not overlap scales", who);
  hipStream_t st = as_stream(stream);
  const long long n_chunks = bytes / 16;
  const uint32_t* src = static_cast<const uint32_t*>(w);
  uint32_t* dst = static_cast<uint32_t*>(w_tiled);
  switch (group_size) {
    case 32:
      hipLaunchKernelGGL((tile_codes_kernel<32, true>), dim3(grid_of(n_chunks)),
                         dim3(kTileThreads), 0, st, src, dst, n_chunks, nblk);
      break;
    case 64:
      hipLaunchKernelGGL((tile_codes_kernel<64, true>), dim3(grid_of(n_chunks)),
                         dim3(kTileThreads), 0, st, src, dst, n_chunks, nblk);
      break;
    case 128:
      hipLaunchKernelGGL((tile_codes_kernel<128, true>), dim3(grid_of(n_chunks)),
                         dim3(kTileThreads), 0, st, src, dst, n_chunks, nblk);
      break;
    default:  // FP16 values: words moved whole
      hipLaunchKernelGGL((tile_codes_kernel<128, false>), dim3(grid_of(n_chunks)),
                         dim3(kTileThreads), 0, st, src, dst, n_chunks, nblk);
  }
  smoe_status s = check_launch(who);
  if (s != SMOE_OK || !int4) return s;
  const uint16_t* ss = static_cast<const uint16_t*>(scales);
  uint16_t* sd = static_cast<uint16_t*>(scales_tiled);
  switch (group_size) {
    case 32:
      hipLaunchKernelGGL(tile_scales_kernel<4>, dim3(grid_of(n_runs)), dim3(kTileThreads), 0, st,
                         ss, sd, n_runs, nblk);
      break;
    case 64:
      hipLaunchKernelGGL(tile_scales_kernel<2>, dim3(grid_of(n_runs)), dim3(kTileThreads), 0, st,
                         ss, sd, n_runs, nblk);
      break;
    default:
      hipLaunchKernelGGL(tile_scales_kernel<1>, dim3(grid_of(n_runs)), dim3(kTileThreads), 0, st,
                         ss, sd, n_runs, nblk);
  }
  return check_launch(who);
}
