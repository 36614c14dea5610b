// Decode kernel (M <= 64): Y = X (deq(Q_base) + deq(R))^T, fused.
//
// ZipperEngine (MosaicQuant explainer, Methodology section 3) runs the sparse
// residual inside the dense 4-bit GEMM kernel so activations are read once and
// no partial outputs are merged by a second kernel. This MI355X version:
//   * one workgroup per 16-row block, KSPLIT waves splitting the column tiles;
//   * each lane streams 16 B of codes per 1 KiB tile (one coalesced 1 KiB
//     wave load per tile), widens them to fp16 s*q in registers and feeds
//     4 MFMA 16x16x32 steps, with X^T as the B operand (tokens as columns);
//   * the residual entries of the wave's tiles are applied in chunks of 32 as
//     one more MFMA each: A is one-hot by row carrying the fp16 corrections,
//     B gathers the matching X columns -- the residual lands in the same fp32
//     accumulators as the base, so nothing is written twice;
//   * the KSPLIT partial tiles are summed in LDS in a fixed order.
#include "kernel_common.h"
#include "mq_internal.h"

namespace mq {
namespace {

template <int MB, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void k_gemv(const uint4* __restrict__ tiles,
                                                      const uint16_t* __restrict__ scales, int64_t sstride,
                                                      const uint32_t* __restrict__ tile_ptr,
                                                      const uint32_t* __restrict__ entries,
                                                      const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                      int M, int N, int K, int G, int Kt) {
  __shared__ float4_t red[KSPLIT][MB][64];
  const int rb = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int row = rb * kRowsPerBlock + r;
  const int kt0 = (Kt * wave) / KSPLIT, kt1 = (Kt * (wave + 1)) / KSPLIT;
  const uint4* tile_base = tiles + (int64_t)rb * Kt * 64 + lane;

  float4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int kt = kt0; kt < kt1; ++kt) {
    const uint4 code = tile_base[(int64_t)kt * 64];
    const int c0 = kt * kTileCols + 32 * g;
    const bool cvalid = c0 < K;
    const uint32_t sb = (cvalid && row < N) ? scales[(int64_t)row * sstride + c0 / G] : 0u;
    const half2_t s2 = splat_half(sb);
    half8_t a[4];
    a[0] = dequant_dword(code.x, s2);
    a[1] = dequant_dword(code.y, s2);
    a[2] = dequant_dword(code.z, s2);
    a[3] = dequant_dword(code.w, s2);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + r;
      uint4 xv[4];
      if (cvalid && m < M) {
        const uint4* xp = reinterpret_cast<const uint4*>(X + (int64_t)m * K + c0);
#pragma unroll
        for (int t = 0; t < 4; ++t) xv[t] = xp[t];
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) xv[t] = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mb] = mfma16(a[t], as_half8(xv[t]), acc[mb]);
    }
  }

  // Residual: entries of tiles [kt0, kt1), one 4096-column window at a time.
  if (kt1 > kt0) {
    for (int win = kt0 >> 5; win <= (kt1 - 1) >> 5; ++win) {
      const int ta = max(kt0, win << 5), tb = min(kt1, (win + 1) << 5);
      const uint32_t eb = tile_ptr[(int64_t)rb * Kt + ta], ee = tile_ptr[(int64_t)rb * Kt + tb];
      const int wbase = win * kColWindow;
      for (uint32_t cb = eb; cb < ee; cb += 32) {
        uint32_t ent[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t idx = cb + 8 * g + u;
          ent[u] = (idx < ee) ? entries[idx] : 0u;   // entry 0 carries a zero correction
        }
        u32x4_t av;
        uint32_t* ap = reinterpret_cast<uint32_t*>(&av);
#pragma unroll
        for (int u = 0; u < 8; u += 2) {
          const uint32_t lo = (ent_row(ent[u]) == (uint32_t)r) ? ent_delta(ent[u]) : 0u;
          const uint32_t hi = (ent_row(ent[u + 1]) == (uint32_t)r) ? ent_delta(ent[u + 1]) : 0u;
          ap[u >> 1] = lo | (hi << 16);
        }
        const half8_t a = __builtin_bit_cast(half8_t, av);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = mb * 16 + r;
          u32x4_t bv;
          uint32_t* bp = reinterpret_cast<uint32_t*>(&bv);
#pragma unroll
          for (int u = 0; u < 8; u += 2) {
            uint32_t lo = 0u, hi = 0u;
            if (m < M) {
              const uint16_t* xr = X + (int64_t)m * K + wbase;
              lo = xr[ent_col(ent[u])];
              hi = xr[ent_col(ent[u + 1])];
            }
            bp[u >> 1] = lo | (hi << 16);
          }
          acc[mb] = mfma16(a, __builtin_bit_cast(half8_t, bv), acc[mb]);
        }
      }
    }
  }

  // Fixed-order sum of the KSPLIT partial tiles, then fp16 output.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float4_t s = red[0][mb][lane];
#pragma unroll
      for (int w = 1; w < KSPLIT; ++w) s += red[w][mb][lane];
      const int m = mb * 16 + r;                   // token
      const int n0 = rb * kRowsPerBlock + 4 * g;   // first of 4 output features
      if (m < M) {
        uint16_t* yp = Y + (int64_t)m * N + n0;
        if (n0 + 3 < N && (N & 3) == 0) {
          const uint32_t lo = (uint32_t)f32_to_h(s.x) | ((uint32_t)f32_to_h(s.y) << 16);
          const uint32_t hi = (uint32_t)f32_to_h(s.z) | ((uint32_t)f32_to_h(s.w) << 16);
          *reinterpret_cast<uint2*>(yp) = make_uint2(lo, hi);
        } else {
          if (n0 + 0 < N) yp[0] = f32_to_h(s.x);
          if (n0 + 1 < N) yp[1] = f32_to_h(s.y);
          if (n0 + 2 < N) yp[2] = f32_to_h(s.z);
          if (n0 + 3 < N) yp[3] = f32_to_h(s.w);
        }
      }
    }
  }
}

template <int MB>
hipError_t run(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  constexpr int KSPLIT = 4;
  k_gemv<MB, KSPLIT><<<dim3((unsigned)p->Nb), dim3(64 * KSPLIT), 0, s>>>(
      reinterpret_cast<const uint4*>(p->tiles), p->scales, p->sstride, p->tile_ptr, p->entries, X, Y, M,
      (int)p->N, (int)p->K, p->G, (int)p->Kt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (M <= 16) return run<1>(p, X, (int)M, Y, s);
  if (M <= 32) return run<2>(p, X, (int)M, Y, s);
  return run<4>(p, X, (int)M, Y, s);
}

}  // namespace mq
