// Prefill kernel (any M): Y = X (deq(Q_base) + deq(R))^T, fused.
//
// ZipperEngine (MosaicQuant explainer, Methodology section 3) runs the sparse
// residual inside the dense 4-bit GEMM so X is read once and no partial
// outputs are merged afterwards. Here the residual is folded into the dense
// weight tile before the matrix cores consume it:
//   * a workgroup of 4 waves computes a 256 (output features) x 256 (tokens)
//     tile, each wave a 128 x 128 block of 8 x 8 16x16x32 fp16 MFMAs with
//     fp32 accumulators;
//   * K advances in stages of 64 columns (half a code tile), double-buffered
//     in LDS: the weight stage is widened from the 4-bit tiles to fp16(s q)
//     by the wave that owns those 4 row blocks, which then patches the
//     stage's residual entries into it (fp16(s q + sr qr), rounded once) --
//     a wave's LDS operations execute in order, so no barrier is needed
//     between its writes and its patches; X is staged through registers;
//   * while a stage's MFMAs run, the next stage is widened, written and
//     patched into the other buffer and the tile after that is requested
//     from memory: one barrier per stage;
//   * workgroups are ordered so that consecutive tiles of one 256-token
//     slice run on the same XCD and share its L2 for X.
#include "kernel_common.h"
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int BN = 256;               // output features per workgroup (16 row blocks)
constexpr int BM = 256;               // tokens per workgroup
constexpr int BK = 64;                // K columns per LDS stage
constexpr int LDW = BK + 8;           // LDS row (halves): 144 B, so 8 consecutive rows hit distinct banks
constexpr int kThreads = 256;
constexpr int kRbPerWave = 4;         // row blocks widened and patched by each wave
constexpr size_t kStageHalves = (size_t)(BN + BM) * LDW;
constexpr size_t kLdsBytes = 2 * kStageHalves * sizeof(_Float16) + (size_t)BN * 2 * sizeof(uint32_t);

// Registers holding one code tile (two stages) of the wave's 4 row blocks.
struct TileRegs {
  uint4 code[kRbPerWave];
  uint2 sraw[kRbPerWave];        // fp16 scales of the lane's row: 1, 2 or 4 groups of the tile
  uint32_t ent[kRbPerWave];      // residual entry p0 + lane of the tile's segment (0 = none)
  uint32_t p0[kRbPerWave], p1[kRbPerWave];
};

template <int GSH>
__device__ __forceinline__ void load_tile(TileRegs& T, const uint4* __restrict__ tiles,
                                          const uint16_t* __restrict__ scales, int64_t sstride,
                                          const uint32_t* __restrict__ tile_ptr,
                                          const uint32_t* __restrict__ entries, int Kt, int Nb, int rbw, int kt,
                                          int lane) {
  const int r = lane & 15;
#pragma unroll
  for (int j = 0; j < kRbPerWave; ++j) {
    const int rb = rbw + j;
    if (rb < Nb && kt < Kt) {
      const int64_t t = (int64_t)rb * Kt + kt;
      T.code[j] = tiles[t * 64 + lane];
      const uint16_t* sp = scales + (int64_t)(rb * kRowsPerBlock + r) * sstride + (kt << GSH);
      if constexpr (GSH == 0) T.sraw[j] = make_uint2(*sp, 0u);
      else if constexpr (GSH == 1) T.sraw[j] = make_uint2(*reinterpret_cast<const uint32_t*>(sp), 0u);
      else T.sraw[j] = *reinterpret_cast<const uint2*>(sp);
      T.p0[j] = tile_ptr[t];
      T.p1[j] = tile_ptr[t + 1];
      T.ent[j] = (T.p0[j] + lane < T.p1[j]) ? entries[T.p0[j] + lane] : 0u;
    } else {
      T.code[j] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
      T.sraw[j] = make_uint2(0u, 0u);
      T.p0[j] = T.p1[j] = 0u;
      T.ent[j] = 0u;
    }
  }
}

// fp16 bits of the scale of dword t (0..3) of the tile.
template <int GSH>
__device__ __forceinline__ uint32_t dword_scale(uint2 sraw, int t) {
  if constexpr (GSH == 0) return sraw.x & 0xFFFFu;
  else if constexpr (GSH == 1) return (sraw.x >> (16 * (t >> 1))) & 0xFFFFu;
  else return ((t < 2 ? sraw.x : sraw.y) >> (16 * (t & 1))) & 0xFFFFu;
}

// X stage [BM tokens][BK columns]: 8 x 16 B per thread, 8 consecutive chunks of a row per 8 lanes.
__device__ __forceinline__ void load_x(uint4 (&x)[8], const uint16_t* __restrict__ X, int M, int K, int m0, int col0,
                                       int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx >> 3, col = col0 + 8 * (idx & 7);
    x[i] = (m0 + row < M && col < K) ? *reinterpret_cast<const uint4*>(X + (int64_t)(m0 + row) * K + col)
                                      : make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ void store_x(const uint4 (&x)[8], _Float16* Xs, int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = tid + kThreads * i;
    *reinterpret_cast<uint4*>(Xs + (idx >> 3) * LDW + 8 * (idx & 7)) = x[i];
  }
}

// Widen half h of the tile (dwords 2h, 2h+1) of the wave's row blocks to fp16(s q)
// in the stage buffer, record the rows' stage scale, then patch the residual
// entries of that half: fp16(s q + sr qr), with q recovered exactly from the
// fp16(s q) just written (|q| <= 7).
template <int GSH>
__device__ __forceinline__ void write_w(const TileRegs& T, _Float16* Ws, uint32_t* ssc, int lrb0, int h, int lane,
                                        const uint32_t* __restrict__ entries) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < kRbPerWave; ++j) {
    _Float16* dst = Ws + ((lrb0 + j) * kRowsPerBlock + r) * LDW + 8 * g;
    const uint32_t d0 = h ? T.code[j].z : T.code[j].x;
    const uint32_t d1 = h ? T.code[j].w : T.code[j].y;
    const uint32_t s0 = dword_scale<GSH>(T.sraw[j], 2 * h), s1 = dword_scale<GSH>(T.sraw[j], 2 * h + 1);
    *reinterpret_cast<half8_t*>(dst) = dequant_dword(d0, splat_half(s0));
    *reinterpret_cast<half8_t*>(dst + 32) = dequant_dword(d1, splat_half(s1));
    if (g == 0) ssc[(lrb0 + j) * kRowsPerBlock + r] = s0 | (s1 << 16);
  }
#pragma unroll
  for (int j = 0; j < kRbPerWave; ++j) {
    for (uint32_t e = T.p0[j] + lane, first = 1; e < T.p1[j]; e += 64, first = 0) {
      const uint32_t v = first ? T.ent[j] : entries[e];
      const int c = (int)(ent_col(v) & (kTileCols - 1));
      if (v == 0u || (c >> 6) != h) continue;   // zero padding, or the other half of the tile
      const int row = (lrb0 + j) * kRowsPerBlock + (int)ent_row(v);
      const uint32_t sb = ssc[row];
      const float s = h_to_f(((c & 63) < 32 ? sb : sb >> 16) & 0xFFFFu);
      _Float16* w = Ws + row * LDW + (c & 63);
      const float q = (s != 0.f) ? rintf((float)*w / s) : 0.f;
      *w = (_Float16)fmaf(s, q, h_to_f(ent_delta(v)));
    }
  }
}

// Tile index of workgroup b: the hardware deals workgroups to the 8 XCDs in
// turn, so the tiles of XCD x are made a contiguous range (one or a few
// token slices, all their feature tiles).
__device__ __forceinline__ int xcd_tile(int b, int T) {
  const int per = T >> 3, rem = T & 7, x = b & 7, local = b >> 3;
  return x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}

template <int GSH>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(const uint4* __restrict__ tiles,
                                                      const uint16_t* __restrict__ scales, int64_t sstride,
                                                      const uint32_t* __restrict__ tile_ptr,
                                                      const uint32_t* __restrict__ entries,
                                                      const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                      int M, int N, int K, int Kt, int Nb, int NT, int T) {
  extern __shared__ __attribute__((aligned(16))) _Float16 lds[];
  uint32_t* const ssc = reinterpret_cast<uint32_t*>(lds + 2 * kStageHalves);   // [2][BN] stage scales

  const int tile = xcd_tile(blockIdx.x, T);
  const int mt = tile / NT, nt = tile - mt * NT;
  const int rb0 = nt * (BN / kRowsPerBlock), m0 = mt * BM;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, tid = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;   // 2 x 2 waves of 128 x 128
  const int lrb0 = kRbPerWave * wave;        // local row blocks widened by this wave
  const int S = 2 * Kt;                      // stages

  float4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  TileRegs cur, nxt;
  uint4 xr[8];
  load_tile<GSH>(cur, tiles, scales, sstride, tile_ptr, entries, Kt, Nb, rb0 + lrb0, 0, lane);
  load_x(xr, X, M, K, m0, 0, tid);
  write_w<GSH>(cur, lds, ssc, lrb0, 0, lane, entries);
  store_x(xr, lds + BN * LDW, tid);
  load_tile<GSH>(nxt, tiles, scales, sstride, tile_ptr, entries, Kt, Nb, rb0 + lrb0, 1, lane);
  load_x(xr, X, M, K, m0, BK, tid);
  __syncthreads();

  for (int s = 0; s < S; ++s) {
    const int b = s & 1;
    const _Float16* Ws = lds + b * kStageHalves;
    const _Float16* Xs = Ws + BN * LDW;
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      half8_t a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        a[i] = *reinterpret_cast<const half8_t*>(Ws + (128 * wn + 16 * i + r) * LDW + 32 * kk + 8 * g);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const half8_t bx = *reinterpret_cast<const half8_t*>(Xs + (128 * wm + 16 * j + r) * LDW + 32 * kk + 8 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i][j] = mfma16(a[i], bx, acc[i][j]);
      }
    }
    if (s + 1 < S) {
      // stage s + 1 into the other buffer (its last readers passed the previous barrier)
      _Float16* Wn = lds + (b ^ 1) * kStageHalves;
      if (s & 1) {          // stage s + 1 starts tile (s + 1) / 2, held in nxt
        write_w<GSH>(nxt, Wn, ssc + (b ^ 1) * BN, lrb0, 0, lane, entries);
        cur = nxt;
        load_tile<GSH>(nxt, tiles, scales, sstride, tile_ptr, entries, Kt, Nb, rb0 + lrb0, (s + 3) >> 1, lane);
      } else {              // second half of the current tile
        write_w<GSH>(cur, Wn, ssc + (b ^ 1) * BN, lrb0, 1, lane, entries);
      }
      store_x(xr, Wn + BN * LDW, tid);
      if (s + 2 < S) load_x(xr, X, M, K, m0, (s + 2) * BK, tid);
    }
    __syncthreads();
  }

  // Epilogue: lane holds D[4 g + q][r] of each 16x16 block -> Y[m][n .. n+3].
  const int nbase = rb0 * kRowsPerBlock + 128 * wn;
  const int mbase = m0 + 128 * wm;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = mbase + 16 * j + r;
      const int n0 = nbase + 16 * i + 4 * g;
      if (m >= M || n0 >= N) continue;
      store4(Y + (int64_t)m * N + n0, acc[i][j], N - n0, (N & 3) == 0);
    }
  }
}

template <int GSH>
hipError_t launch(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<GSH>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int NT = (int)((p->Nb + (BN / kRowsPerBlock) - 1) / (BN / kRowsPerBlock));
  const int MT = (int)((M + BM - 1) / BM);
  const int T = NT * MT;
  k_gemm<GSH><<<dim3((unsigned)T), dim3(kThreads), kLdsBytes, s>>>(
      reinterpret_cast<const uint4*>(p->tiles), p->scales, p->sstride, p->tile_ptr, p->entries, X, Y, (int)M,
      (int)p->N, (int)p->K, (int)p->Kt, (int)p->Nb, NT, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (p->G == 128) return launch<0>(p, X, M, Y, s);
  if (p->G == 64) return launch<1>(p, X, M, Y, s);
  return launch<2>(p, X, M, Y, s);
}

}  // namespace mq
