// Prefill kernel (any M): Y = X (deq(Q_base) + deq(R))^T, fused.
//
// Per 128-column tile (one code tile) a workgroup of 256 threads
//   1. widens 8 code tiles (128 output features) to fp16 s*q and stores them
//      in LDS, and stages the 128x128 fp16 block of X in LDS;
//   2. applies the tile's residual entries in LDS: each entry adds its fp16
//      correction to the one weight it patches (entries are unique, so no two
//      lanes touch the same 16-bit word);
//   3. runs 16x16x32 fp16 MFMAs with fp32 accumulation from LDS, while the
//      next tile's codes and X are already in flight (double-buffered LDS).
// This is the ZipperEngine's fused dense + sparse schedule (MosaicQuant
// explainer, Methodology section 3) with the sparse part folded into the
// dense operand before the matrix cores consume it.
#include "kernel_common.h"
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int BN = 128;            // output features per workgroup (8 row blocks)
constexpr int BM = 128;            // tokens per workgroup
constexpr int LDK = kTileCols + 8; // padded LDS row (halves) against bank conflicts
constexpr int kThreads = 256;
constexpr size_t kLdsBytes = 2ull * (BN + BM) * LDK * sizeof(_Float16);

struct StageRegs {
  uint4 code[2];
  uint32_t sbits[2][4];   // scale of each dword (32-column segment) of the lane
  uint4 x[8];
};

__device__ __forceinline__ void load_stage(StageRegs& R, const uint4* __restrict__ tiles,
                                           const uint16_t* __restrict__ scales, int64_t sstride,
                                           const uint16_t* __restrict__ X, int M, int N, int K, int G, int Kt,
                                           int Nb, int rb0, int m0, int kt, int wave, int lane) {
  const int r = lane & 15;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rb = rb0 + 2 * wave + j;
    const int row = rb * kRowsPerBlock + r;
    if (rb < Nb) {
      R.code[j] = tiles[((int64_t)rb * Kt + kt) * 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {   // dword t covers columns 128 kt + 32 t + ...
        const int seg = kt * kTileCols + 32 * t;
        R.sbits[j][t] = (row < N && seg < K) ? scales[(int64_t)row * sstride + seg / G] : 0u;
      }
    } else {
      R.code[j] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
#pragma unroll
      for (int t = 0; t < 4; ++t) R.sbits[j][t] = 0u;
    }
  }
  const int tid = wave * 64 + lane;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = tid + kThreads * i;
    const int xr = idx >> 4, xc = idx & 15;
    const int m = m0 + xr, col = kt * kTileCols + 8 * xc;
    R.x[i] = (m < M && col < K) ? *reinterpret_cast<const uint4*>(X + (int64_t)m * K + col)
                                : make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ void store_stage(const StageRegs& R, _Float16* Ws, _Float16* Xs, int wave, int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // dword t of lane (r, g) holds columns 32 t + 8 g + 0..7 of its row
    _Float16* dst = Ws + ((2 * wave + j) * kRowsPerBlock + r) * LDK + 8 * g;
    const uint32_t d[4] = {R.code[j].x, R.code[j].y, R.code[j].z, R.code[j].w};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      *reinterpret_cast<half8_t*>(dst + 32 * t) = dequant_dword(d[t], splat_half(R.sbits[j][t]));
  }
  const int tid = wave * 64 + lane;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = tid + kThreads * i;
    const int xr = idx >> 4, xc = idx & 15;
    *reinterpret_cast<uint4*>(Xs + xr * LDK + 8 * xc) = R.x[i];
  }
}

// Residual entries of the stage: the weight becomes fp16(s q + sr qr), rounded
// once. q is read back from the widened fp16(s q) in LDS (|q| <= 7, so
// rint(fp16(s q) / s) recovers it exactly), s from the scale table.
__device__ __forceinline__ void patch_stage(_Float16* Ws, const uint32_t* __restrict__ tile_ptr,
                                            const uint32_t* __restrict__ entries,
                                            const uint16_t* __restrict__ scales, int64_t sstride, int gshift,
                                            int N, int Nb, int Kt, int rb0, int kt, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rb = rb0 + 2 * wave + j;
    if (rb >= Nb) continue;
    const uint32_t p0 = tile_ptr[(int64_t)rb * Kt + kt], p1 = tile_ptr[(int64_t)rb * Kt + kt + 1];
    for (uint32_t e = p0 + lane; e < p1; e += 64) {
      const uint32_t v = entries[e];
      if (v == 0u) continue;   // zero padding (a real entry that encodes to 0 changes nothing)
      const int row = rb * kRowsPerBlock + (int)ent_row(v);
      const int kk = (int)(ent_col(v) & (kTileCols - 1));
      const float s = h_to_f(scales[(int64_t)row * sstride + ((kt * kTileCols + kk) >> gshift)]);
      _Float16* w = Ws + ((2 * wave + j) * kRowsPerBlock + (int)ent_row(v)) * LDK + kk;
      const float q = (s != 0.f) ? rintf((float)*w / s) : 0.f;
      *w = (_Float16)fmaf(s, q, h_to_f(ent_delta(v)));
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_gemm(const uint4* __restrict__ tiles,
                                                   const uint16_t* __restrict__ scales, int64_t sstride,
                                                   const uint32_t* __restrict__ tile_ptr,
                                                   const uint32_t* __restrict__ entries,
                                                   const uint16_t* __restrict__ X, uint16_t* __restrict__ Y, int M,
                                                   int N, int K, int G, int Kt, int Nb) {
  const int gshift = (G == 128) ? 7 : (G == 64) ? 6 : 5;
  extern __shared__ __attribute__((aligned(16))) _Float16 lds[];
  // buffer b: weights at lds + b * BN * LDK, activations after both weight buffers
  _Float16* const Wlds = lds;
  _Float16* const Xlds = lds + 2 * BN * LDK;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int rb0 = blockIdx.x * (BN / kRowsPerBlock);
  const int m0 = blockIdx.y * BM;
  const int wn = wave & 1, wm = wave >> 1;   // 2 x 2 waves, 64 x 64 outputs each

  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  StageRegs R;
  load_stage(R, tiles, scales, sstride, X, M, N, K, G, Kt, Nb, rb0, m0, 0, wave, lane);
  store_stage(R, Wlds, Xlds, wave, lane);
  __syncthreads();
  patch_stage(Wlds, tile_ptr, entries, scales, sstride, gshift, N, Nb, Kt, rb0, 0, wave, lane);
  __syncthreads();

  for (int kt = 0; kt < Kt; ++kt) {
    const int b = kt & 1;
    const bool more = kt + 1 < Kt;
    if (more) load_stage(R, tiles, scales, sstride, X, M, N, K, G, Kt, Nb, rb0, m0, kt + 1, wave, lane);
    const _Float16* Ws = Wlds + b * BN * LDK;
    const _Float16* Xs = Xlds + b * BM * LDK;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      half8_t a[4], bx[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const half8_t*>(Ws + (64 * wn + 16 * i + r) * LDK + 32 * t + 8 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bx[j] = *reinterpret_cast<const half8_t*>(Xs + (64 * wm + 16 * j + r) * LDK + 32 * t + 8 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[i], bx[j], acc[i][j]);
    }
    if (more) {
      store_stage(R, Wlds + (b ^ 1) * BN * LDK, Xlds + (b ^ 1) * BM * LDK, wave, lane);
      __syncthreads();
      patch_stage(Wlds + (b ^ 1) * BN * LDK, tile_ptr, entries, scales, sstride, gshift, N, Nb, Kt, rb0, kt + 1,
                  wave, lane);
    }
    __syncthreads();
  }

  // Epilogue: lane holds D[4 g + q][r] of each 16x16 block -> Y[m][n .. n+3].
  const int nbase = rb0 * kRowsPerBlock + 64 * wn;
  const int mbase = m0 + 64 * wm;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = mbase + 16 * j + r;
      const int n0 = nbase + 16 * i + 4 * g;
      if (m >= M) continue;
      const float4_t s = acc[i][j];
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

}  // namespace

hipError_t launch_gemm(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned nt = (unsigned)((p->Nb + (BN / kRowsPerBlock) - 1) / (BN / kRowsPerBlock));
  const unsigned mt = (unsigned)((M + BM - 1) / BM);
  k_gemm<<<dim3(nt, mt), dim3(kThreads), kLdsBytes, s>>>(reinterpret_cast<const uint4*>(p->tiles), p->scales,
                                                          p->sstride, p->tile_ptr, p->entries, X, Y, (int)M,
                                                          (int)p->N, (int)p->K, p->G, (int)p->Kt, (int)p->Nb);
  return hipGetLastError();
}

}  // namespace mq
