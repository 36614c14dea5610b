// Prefill kernel (any M): Y = X (deq(Q_base) + deq(R))^T, fused.
//
// ZipperEngine (MosaicQuant explainer, Methodology section 3) runs the sparse
// residual inside the dense 4-bit GEMM so X is read once and no partial
// outputs are merged afterwards. Here the residual is folded into the dense
// weight tile before the matrix cores consume it:
//   * a workgroup of 4 waves computes a 256 (output features) x 256 (tokens)
//     tile, each wave a 128 x 128 block of 4 x 4 32x32x16 fp16 MFMAs with
//     fp32 accumulators;
//   * K advances in stages of 64 columns (half a code tile), double-buffered
//     in LDS: the weight stage is widened from the 4-bit tiles to fp16(s q)
//     by the wave that owns those 4 row blocks, which then patches the
//     stage's residual entries into it (fp16(s q + sr qr), rounded once) --
//     a wave's LDS operations execute in order, so no barrier is needed
//     between its writes and its patches; X is staged through registers;
//   * one loop iteration is one code tile (two stages); its body has no
//     branches, so the widening, patching and X staging of the next stage
//     interleave with the current stage's MFMAs; one barrier per stage;
//   * workgroups are ordered so that consecutive tiles of one 256-token
//     slice run on the same XCD and share its L2 for X.
#include "kernel_common.h"
#include "mq_internal.h"

namespace mq {
namespace {

typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int BN = 256;               // output features per workgroup (16 row blocks)
constexpr int BM = 256;               // tokens per workgroup
constexpr int BK = 64;                // K columns per LDS stage
constexpr int LDW = BK + 8;           // LDS row (halves): 144 B, so 8 consecutive rows hit distinct banks
constexpr int kThreads = 256;
constexpr int kRbPerWave = 4;         // row blocks widened and patched by each wave
constexpr size_t kStageHalves = (size_t)(BN + BM) * LDW;
constexpr size_t kScaleOff = 2 * kStageHalves * sizeof(_Float16);             // [2][BN] u32 stage scales
constexpr size_t kDummyOff = kScaleOff + 2 * BN * sizeof(uint32_t);            // patch target of idle lanes
constexpr size_t kLdsBytes = kDummyOff + 16;

// Registers holding one code tile (two stages) of the wave's 4 row blocks.
struct TileRegs {
  uint4 code[kRbPerWave];
  uint2 sraw[kRbPerWave];        // fp16 scales of the lane's row: 1, 2 or 4 groups of the tile
  uint32_t ent[kRbPerWave];      // residual entry p0 + lane of the tile's segment (0 = none)
  uint32_t p0[kRbPerWave], cnt[kRbPerWave];
};

// Branch-free: a row block past the layer or a tile past K reads clamped
// indices and yields codes of q = 0, scale 0 and no entries. Entry loads stay
// in bounds because 1024 zero entries follow the stream.
template <int GSH>
__device__ __forceinline__ void load_tile(TileRegs& T, const uint4* __restrict__ tiles,
                                          const uint16_t* __restrict__ scales, int64_t sstride,
                                          const uint32_t* __restrict__ tile_ptr,
                                          const uint32_t* __restrict__ entries, int Kt, int Nb, int rbw, int kt,
                                          int lane) {
  const int r = lane & 15;
#pragma unroll
  for (int j = 0; j < kRbPerWave; ++j) {
    const bool ok = rbw + j < Nb && kt < Kt;
    const int rb = min(rbw + j, Nb - 1), ktc = min(kt, Kt - 1);
    const int64_t t = (int64_t)rb * Kt + ktc;
    const uint4 c = tiles[t * 64 + lane];
    const uint16_t* sp = scales + (int64_t)(rb * kRowsPerBlock + r) * sstride + (ktc << GSH);
    uint2 sr;
    if constexpr (GSH == 0) sr = make_uint2(*sp, 0u);
    else if constexpr (GSH == 1) sr = make_uint2(*reinterpret_cast<const uint32_t*>(sp), 0u);
    else sr = *reinterpret_cast<const uint2*>(sp);
    const uint32_t p0 = tile_ptr[t], p1 = tile_ptr[t + 1];
    const uint32_t e = entries[p0 + lane];
    T.code[j] = ok ? c : make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
    T.sraw[j] = ok ? sr : make_uint2(0u, 0u);
    T.p0[j] = p0;
    T.cnt[j] = ok ? p1 - p0 : 0u;
    T.ent[j] = (uint32_t)lane < T.cnt[j] ? e : 0u;
  }
}

// fp16 bits of the scale of dword t (0..3) of the tile.
template <int GSH>
__device__ __forceinline__ uint32_t dword_scale(uint2 sraw, int t) {
  if constexpr (GSH == 0) return sraw.x & 0xFFFFu;
  else if constexpr (GSH == 1) return (sraw.x >> (16 * (t >> 1))) & 0xFFFFu;
  else return ((t < 2 ? sraw.x : sraw.y) >> (16 * (t & 1))) & 0xFFFFu;
}

// X stage [BM tokens][BK columns]: 8 x 16 B per thread, 8 consecutive chunks of a
// row per 8 lanes; thread tid reads rows tid / 8 + 32 i, chunk tid % 8, so its
// 8 row pointers are fixed (xrow, computed once; rows past M read row M - 1,
// which only feeds outputs that are never stored). Every load is
// unconditional (a guarded load would become a branch); when K is not a
// multiple of 128 the chunks past K are zeroed with a mask kept opaque to the
// compiler (a select would be turned back into a branch).
template <bool KTAIL>
__device__ __forceinline__ void load_x(uint4 (&x)[8], const uint16_t* const (&xrow)[8], int K, int col0, int tid) {
  // without a K tail (K % 128 == 0) only the look-ahead past the last stage
  // leaves [0, K): it re-reads the last stage (never consumed)
  const int col = (KTAIL ? col0 : min(col0, K - BK)) + 8 * (tid & 7);
  uint32_t keep = col < K ? ~0u : 0u;
  if (KTAIL) asm volatile("" : "+v"(keep));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(xrow[i] + (KTAIL ? min(col, K - 8) : col));
    x[i] = KTAIL ? make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep) : v;
  }
}

__device__ __forceinline__ void store_x(const uint4 (&x)[8], _Float16* Xs, int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = tid + kThreads * i;
    *reinterpret_cast<uint4*>(Xs + (idx >> 3) * LDW + 8 * (idx & 7)) = x[i];
  }
}

// Widen half h of the tile (dwords 2h, 2h+1) of the wave's row blocks to
// fp16(s q) in the stage buffer, record each row's stage scales, then patch
// the first 64 residual entries of each tile segment that fall in this half:
// fp16(s q + sr qr), with q recovered exactly from the fp16(s q) just written
// (|q| <= 7, so any reciprocal within a few ulp gives the right rint). Lanes
// without an entry write to a dummy word (no branches).
template <int GSH>
__device__ __forceinline__ void write_w(const TileRegs& T, _Float16* Ws, uint32_t* ssc, _Float16* dummy, int lrb0,
                                        int h, int lane, uint32_t vmask, uint32_t vmask4, uint32_t vmagic) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < kRbPerWave; ++j) {
    _Float16* dst = Ws + ((lrb0 + j) * kRowsPerBlock + r) * LDW + 8 * g;
    const uint32_t d0 = h ? T.code[j].z : T.code[j].x;
    const uint32_t d1 = h ? T.code[j].w : T.code[j].y;
    const uint32_t s0 = dword_scale<GSH>(T.sraw[j], 2 * h), s1 = dword_scale<GSH>(T.sraw[j], 2 * h + 1);
    *reinterpret_cast<half8_t*>(dst) = dequant_dword(d0, splat_half(s0), vmask, vmask4, vmagic);
    *reinterpret_cast<half8_t*>(dst + 32) = dequant_dword(d1, splat_half(s1), vmask, vmask4, vmagic);
    ssc[(lrb0 + j) * kRowsPerBlock + r] = s0 | (s1 << 16);   // same value from the 4 lanes of a row
  }
#pragma unroll
  for (int j = 0; j < kRbPerWave; ++j) {
    const uint32_t v = T.ent[j];
    const int c = (int)(ent_col(v) & (kTileCols - 1));
    const bool ok = v != 0u && (c >> 6) == h;
    const int row = (lrb0 + j) * kRowsPerBlock + (int)ent_row(v);
    const uint32_t sb = ssc[row];
    const float s = h_to_f(((c & 63) < 32 ? sb : sb >> 16) & 0xFFFFu);
    _Float16* w = ok ? Ws + row * LDW + (c & 63) : dummy;
    // s = 0 means fp16(s q) = 0, and then q = rint(0 * 1e30) = 0 as well: no select
    const float q = rintf((float)*w * __builtin_amdgcn_rcpf(fmaxf(s, 1e-30f)));
    *w = (_Float16)fmaf(s, q, h_to_f(ent_delta(v)));
  }
}

// Entries 64.. of tile segments longer than 64 (dense residual tiles): rare.
template <int GSH>
__device__ __forceinline__ void patch_rest(const TileRegs& T, _Float16* Ws, const uint32_t* ssc, int lrb0, int h,
                                        int lane, const uint32_t* __restrict__ entries) {
  for (int j = 0; j < kRbPerWave; ++j) {
    for (uint32_t e = T.p0[j] + 64 + lane; e < T.p0[j] + T.cnt[j]; e += 64) {
      const uint32_t v = entries[e];
      const int c = (int)(ent_col(v) & (kTileCols - 1));
      if (v == 0u || (c >> 6) != h) continue;
      const int row = (lrb0 + j) * kRowsPerBlock + (int)ent_row(v);
      const uint32_t sb = ssc[row];
      const float s = h_to_f(((c & 63) < 32 ? sb : sb >> 16) & 0xFFFFu);
      _Float16* w = Ws + row * LDW + (c & 63);
      const float q = (s != 0.f) ? rintf((float)*w * __builtin_amdgcn_rcpf(s)) : 0.f;
      *w = (_Float16)fmaf(s, q, h_to_f(ent_delta(v)));
    }
  }
}

// One stage of MFMAs: wave (wn, wm) multiplies its 128 weight rows by its 128
// token columns over the stage's 64 columns (4 k-steps of 16). Lane l feeds
// row / column l % 32 and k 8 (l / 32) .. +7 of each 32x32x16 step.
__device__ __forceinline__ void mfma_stage(float16_t (&acc)[4][4], const _Float16* Ws, const _Float16* Xs, int wn,
                                           int wm, int lane) {
  const int r32 = lane & 31, kh = 8 * (lane >> 5);
  const _Float16* wa = Ws + (128 * wn + r32) * LDW + kh;
  const _Float16* xb = Xs + (128 * wm + r32) * LDW + kh;
  half8_t a[2][4], b[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[0][i] = *reinterpret_cast<const half8_t*>(wa + 32 * i * LDW);
    b[0][i] = *reinterpret_cast<const half8_t*>(xb + 32 * i * LDW);
  }
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int cb = ks & 1, nb = cb ^ 1;
    if (ks + 1 < BK / 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[nb][i] = *reinterpret_cast<const half8_t*>(wa + 32 * i * LDW + 16 * (ks + 1));
        b[nb][i] = *reinterpret_cast<const half8_t*>(xb + 32 * i * LDW + 16 * (ks + 1));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[cb][i], b[cb][j], acc[i][j], 0, 0, 0);
  }
}

// Tile index of workgroup b: the hardware deals workgroups to the 8 XCDs in
// turn, so the tiles of XCD x are made a contiguous range (one or a few
// token slices, all their feature tiles).
__device__ __forceinline__ int xcd_tile(int b, int T) {
  const int per = T >> 3, rem = T & 7, x = b & 7, local = b >> 3;
  return x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}

template <int GSH, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(const uint4* __restrict__ tiles,
                                                      const uint16_t* __restrict__ scales, int64_t sstride,
                                                      const uint32_t* __restrict__ tile_ptr,
                                                      const uint32_t* __restrict__ entries,
                                                      const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                      int M, int N, int K, int Kt, int Nb, int NT, int T) {
  extern __shared__ __attribute__((aligned(16))) _Float16 lds[];
  uint32_t* const ssc = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(lds) + kScaleOff);
  _Float16* const dummy = reinterpret_cast<_Float16*>(reinterpret_cast<char*>(lds) + kDummyOff);
  _Float16* const buf0 = lds;
  _Float16* const buf1 = lds + kStageHalves;

  const int tile = xcd_tile(blockIdx.x, T);
  const int mt = tile / NT, nt = tile - mt * NT;
  const int rb0 = nt * (BN / kRowsPerBlock), m0 = mt * BM;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, tid = threadIdx.x;
  const int wn = wave & 1, wm = wave >> 1;   // 2 x 2 waves of 128 x 128
  const int lrb0 = kRbPerWave * wave;        // local row blocks widened by this wave
  const int rbw = rb0 + lrb0;
  const uint16_t* xrow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) xrow[i] = X + (int64_t)min(m0 + (tid >> 3) + 32 * i, M - 1) * K;
  uint32_t vmask = 0x000F000Fu, vmask4 = 0x00F000F0u, vmagic = 0x64006400u;
  asm volatile("" : "+v"(vmask), "+v"(vmask4), "+v"(vmagic));   // keep the constants in VGPRs for v_and_or_b32

  float16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  TileRegs t0, t1;
  uint4 xr[8];
  load_tile<GSH>(t0, tiles, scales, sstride, tile_ptr, entries, Kt, Nb, rbw, 0, lane);
  load_x<KTAIL>(xr, xrow, K, 0, tid);
  write_w<GSH>(t0, buf0, ssc, dummy, lrb0, 0, lane, vmask, vmask4, vmagic);
  if (t0.cnt[0] > 64 || t0.cnt[1] > 64 || t0.cnt[2] > 64 || t0.cnt[3] > 64)
    patch_rest<GSH>(t0, buf0, ssc, lrb0, 0, lane, entries);
  store_x(xr, buf0 + BN * LDW, tid);
  load_x<KTAIL>(xr, xrow, K, BK, tid);
  load_tile<GSH>(t1, tiles, scales, sstride, tile_ptr, entries, Kt, Nb, rbw, 1, lane);
  __syncthreads();

  for (int kt = 0; kt < Kt; ++kt) {
    // stage 2 kt (buffer 0) runs; stage 2 kt + 1 (half 1 of tile kt) is prepared in buffer 1
    mfma_stage(acc, buf0, buf0 + BN * LDW, wn, wm, lane);
    write_w<GSH>(t0, buf1, ssc + BN, dummy, lrb0, 1, lane, vmask, vmask4, vmagic);
    store_x(xr, buf1 + BN * LDW, tid);
    load_x<KTAIL>(xr, xrow, K, (2 * kt + 2) * BK, tid);
    if (t0.cnt[0] > 64 || t0.cnt[1] > 64 || t0.cnt[2] > 64 || t0.cnt[3] > 64)
      patch_rest<GSH>(t0, buf1, ssc + BN, lrb0, 1, lane, entries);
    __syncthreads();
    // stage 2 kt + 1 (buffer 1) runs; stage 2 kt + 2 (half 0 of tile kt + 1) is prepared in buffer 0
    mfma_stage(acc, buf1, buf1 + BN * LDW, wn, wm, lane);
    write_w<GSH>(t1, buf0, ssc, dummy, lrb0, 0, lane, vmask, vmask4, vmagic);
    store_x(xr, buf0 + BN * LDW, tid);
    load_x<KTAIL>(xr, xrow, K, (2 * kt + 3) * BK, tid);
    if (t1.cnt[0] > 64 || t1.cnt[1] > 64 || t1.cnt[2] > 64 || t1.cnt[3] > 64)
      patch_rest<GSH>(t1, buf0, ssc, lrb0, 0, lane, entries);
    t0 = t1;
    load_tile<GSH>(t1, tiles, scales, sstride, tile_ptr, entries, Kt, Nb, rbw, kt + 2, lane);
    __syncthreads();
  }

  // Epilogue: register v of lane l holds D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32]
  // of each 32x32 block (rows = output features, columns = tokens).
  const int nbase = rb0 * kRowsPerBlock + 128 * wn + 4 * (lane >> 5);
  const int mbase = m0 + 128 * wm + (lane & 31);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = mbase + 32 * j;
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n0 = nbase + 32 * i + 8 * q;
        if (n0 >= N) continue;
        const float4_t s = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        store4(Y + (int64_t)m * N + n0, s, N - n0, (N & 3) == 0);
      }
    }
  }
}

template <int GSH, bool KTAIL>
hipError_t launch(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<GSH, KTAIL>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int NT = (int)((p->Nb + (BN / kRowsPerBlock) - 1) / (BN / kRowsPerBlock));
  const int MT = (int)((M + BM - 1) / BM);
  const int T = NT * MT;
  k_gemm<GSH, KTAIL><<<dim3((unsigned)T), dim3(kThreads), kLdsBytes, s>>>(
      reinterpret_cast<const uint4*>(p->tiles), p->scales, p->sstride, p->tile_ptr, p->entries, X, Y, (int)M,
      (int)p->N, (int)p->K, (int)p->Kt, (int)p->Nb, NT, T);
  return hipGetLastError();
}

}  // namespace

template <bool KTAIL>
hipError_t launch_k(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (p->G == 128) return launch<0, KTAIL>(p, X, M, Y, s);
  if (p->G == 64) return launch<1, KTAIL>(p, X, M, Y, s);
  return launch<2, KTAIL>(p, X, M, Y, s);
}

hipError_t launch_gemm(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  return (p->K % kTileCols) != 0 ? launch_k<true>(p, X, M, Y, s) : launch_k<false>(p, X, M, Y, s);
}

}  // namespace mq
