// Helpers shared by the packing kernels (pack.hip, pack_blocks.hip): the
// lane <-> tile mapping of a 16 x 128 code tile, exact base errors, and
// wave / workgroup scans.
#pragma once
#include "mq_internal.h"
#include "quant_exact.h"

namespace mq {
namespace pack_detail {

constexpr int kWave = 64;

// Nibble position of column offset c (0..7) inside a dword of the tile layout.
// The fused kernels widen a dword into four fp16 pairs by masking bits 0-3 and
// 16-19, then 4-7 and 20-23, ...; this order makes those pairs hold columns
// (0,1), (2,3), (4,5), (6,7).
__device__ __forceinline__ int nib_pos(int c) { return (c >> 1) + 4 * (c & 1); }

struct LaneTile {
  int row, c0;
  bool valid;
};

__device__ __forceinline__ LaneTile lane_tile(int rb, int kt, int lane, int N, int K) {
  LaneTile t;
  t.row = rb * kRowsPerBlock + (lane & 15);
  t.c0 = kt * kTileCols + 32 * (lane >> 4);
  t.valid = (t.row < N) && (t.c0 < K);
  return t;
}

__device__ __forceinline__ void load32(const uint16_t* __restrict__ W, int64_t K, const LaneTile& t,
                                       uint32_t (&w)[16]) {
  const uint4* src = reinterpret_cast<const uint4*>(W + (int64_t)t.row * K + t.c0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i + 0] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
}

__device__ __forceinline__ uint32_t half_at(const uint32_t (&w)[16], int c) {
  return (w[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
}

__device__ __forceinline__ uint64_t lane_scale_units(const uint16_t* __restrict__ scales, int64_t sstride,
                                                     int G, const LaneTile& t) {
  return (uint64_t)fp16_units(scales[(int64_t)t.row * sstride + t.c0 / G]);
}

// Base errors e = w - s q (units) and their order keys for one lane's 32 entries.
__device__ __forceinline__ void keys_from_w(const uint32_t (&w)[16], uint64_t S, uint64_t (&key)[32],
                                            int64_t (&e)[32]) {
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const int64_t wu = fp16_units(half_at(w, c));
    const int q = quant7(wu, S);
    e[c] = wu - (int64_t)S * q;
    key[c] = err_key((uint64_t)(e[c] < 0 ? -e[c] : e[c]));
  }
}

// Recompute the 32 error keys of one lane (integers |e| * 2^24 as double bits).
__device__ __forceinline__ void lane_keys(const uint16_t* __restrict__ W, const uint16_t* __restrict__ scales,
                                          int64_t K, int G, int64_t sstride, const LaneTile& t,
                                          uint64_t (&key)[32], int64_t (&e)[32]) {
  uint32_t w[16];
  load32(W, K, t, w);
  keys_from_w(w, lane_scale_units(scales, sstride, G, t), key, e);
}

// Inclusive scan of one value per thread over a block of 1024 threads.
__device__ __forceinline__ uint64_t block_scan_incl(uint64_t v, uint64_t* wave_tot) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint64_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == kWave - 1) wave_tot[wave] = v;
  __syncthreads();
  if (wave == 0) {
    uint64_t x = (lane < (int)(blockDim.x / kWave)) ? wave_tot[lane] : 0ull;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const uint64_t u = __shfl_up(x, o);
      if (lane >= o) x += u;
    }
    if (lane < 16) wave_tot[lane] = x;
  }
  __syncthreads();
  const uint64_t base = (wave > 0) ? wave_tot[wave - 1] : 0ull;
  const uint64_t r = v + base;
  __syncthreads();
  return r;
}

// Sum / exclusive prefix of a per-lane value over the four lanes of one row
// (lanes r, r+16, r+32, r+48 hold columns in that order).
__device__ __forceinline__ void row_lanes(uint32_t v, int lane, uint32_t* excl, uint32_t* total) {
  const int r = lane & 15, kq = lane >> 4;
  const uint32_t v0 = __shfl((int)v, r), v1 = __shfl((int)v, r + 16);
  const uint32_t v2 = __shfl((int)v, r + 32), v3 = __shfl((int)v, r + 48);
  *total = v0 + v1 + v2 + v3;
  *excl = (kq > 0 ? v0 : 0u) + (kq > 1 ? v1 : 0u) + (kq > 2 ? v2 : 0u);
}

}  // namespace pack_detail
}  // namespace mq
