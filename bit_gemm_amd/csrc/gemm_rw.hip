// Prefill kernel for long token batches with the weights widened in
// registers: Y = X deq(Q_base)^T, fused.
//
// ZipperEngine (MosaicQuant explainer, Methodology section 3) runs the
// low-bit GEMM as one fused kernel that reads each weight once. On gfx950 the
// fp16 matrix cores outrun the LDS when the widened weights are staged
// through it (every wave that shares a weight row reads it back), so here the
// weights never pass through LDS:
//   * a workgroup of 8 waves (two per SIMD) computes 256 output features x
//     256 tokens; wave (wn, wm) owns 4 row blocks (64 features) and 8 token
//     blocks (128 tokens), 32 accumulator tiles of the 16x16x32 fp16 MFMA
//     in the 128 accumulation registers a wave of two per SIMD has;
//   * K advances one code tile (128 columns) per stage. Each wave loads its
//     4 code tiles straight into registers, a stage ahead, and widens them
//     there to fp16(s q): the tile layout is the A operand as stored. Two
//     waves widen each row block (one per token half), half the widening of
//     a layout that gives every wave all 256 tokens;
//   * X is copied straight from global memory into LDS, a stage ahead, in
//     the B-operand order of the MFMA (quads read 64-byte runs of a token
//     row, and 16 lanes of a B read hit distinct bank groups); a stage's X
//     is 64 KiB, double-buffered, with one barrier per stage;
//   * workgroups are ordered so that the tiles of one 256-token slice run on
//     the same XCD and share its L2 for X.
// Per stage a wave reads 32 KiB of X from LDS for 128 MFMAs, against 24 KiB
// of weights and X for 32 MFMAs when the widened weights are staged in LDS.
#include "kernel_common.h"
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int kWavesW = 8;                                   // two per SIMD
constexpr int kThreadsW = 64 * kWavesW;
constexpr int kRbWave = 4;                                   // row blocks per wave
constexpr int kTbWave = 8;                                   // token blocks per wave
constexpr int kBNW = 4 * kRbWave * kRowsPerBlock;            // 256 output features per workgroup
constexpr int kBMW = 2 * kTbWave * 16;                       // 256 tokens per workgroup
constexpr int kTbCopy = kBMW / 16 / kWavesW;                 // token blocks each wave copies per stage
constexpr int kXBlock = 4096;                                // bytes: one token block's X for one code tile
constexpr int kXStage = (kBMW / 16) * kXBlock;               // 64 KiB
constexpr size_t kLdsW = 2 * (size_t)kXStage;

constexpr uint32_t kSelLoW = 0x05040100u, kSelHiW = 0x07060302u;
__device__ __forceinline__ half2_t splat_sel_w(uint32_t dword, uint32_t sel) {
  return __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dword, dword, sel));
}

// One code tile of the wave's 4 row blocks, loaded a stage ahead: the lane's
// 16 bytes of codes and the aligned scale word(s) of its row holding the
// tile's scale(s). Row blocks past the layer repeat the last (their outputs
// are never stored); rows past N have scale 0.
template <int GSH>
struct WTile {
  uint4 code[kRbWave];
  uint32_t sraw[kRbWave][GSH == 2 ? 2 : 1];
};

// Code tiles and scales come through buffer resources: one per-lane offset
// for all row blocks (the lane's 16 bytes of a tile; its row's scales) and a
// wave-uniform offset per row block, so no per-row-block address takes
// vector registers.
struct WSrc {
  __amdgpu_buffer_rsrc_t tiles, scales;
  uint32_t tl, sl;   // per-lane byte offsets
};

template <int GSH>
__device__ __forceinline__ void w_load(WTile<GSH>& T, const WSrc& S, int64_t sstride, int Kt, int Nb, int rbw, int kt) {
#pragma unroll
  for (int j = 0; j < kRbWave; ++j) {
    const int rb = min(rbw + j, Nb - 1);
    const uint32_t tu = (uint32_t)(rb * Kt + kt) * (uint32_t)kTileBytes;
    const auto c = __builtin_amdgcn_raw_buffer_load_b128(S.tiles, S.tl, tu, 0);
    T.code[j] = make_uint4(c[0], c[1], c[2], c[3]);
    const uint32_t su = (uint32_t)(rb * kRowsPerBlock) * (uint32_t)sstride * 2u;
    if constexpr (GSH == 0) {
      T.sraw[j][0] = __builtin_amdgcn_raw_buffer_load_b32(S.scales, S.sl, su + 4u * (uint32_t)(kt >> 1), 0);
    } else if constexpr (GSH == 1) {
      T.sraw[j][0] = __builtin_amdgcn_raw_buffer_load_b32(S.scales, S.sl, su + 4u * (uint32_t)kt, 0);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(S.scales, S.sl, su + 8u * (uint32_t)kt, 0);
      T.sraw[j][0] = v[0];
      T.sraw[j][1] = v[1];
    }
  }
}

// The X of code tile kt for the workgroup's 256 tokens into one stage buffer:
// wave w copies token blocks 4 w .. 4 w + 3, 4 copies of 1 KiB each, lane
// l's 16 bytes landing at 16 l. The buffer resource spans the workgroup's
// token rows; the whole byte offset (xl: the lane's part) goes into the
// per-lane offset, which its range check covers, so rows past M read zero.
__device__ __forceinline__ void x_copy(uint8_t* buf, __amdgpu_buffer_rsrc_t xr, const uint32_t (&xl)[4], int K,
                                       int kt, int wave) {
#pragma unroll
  for (int i = 0; i < kTbCopy; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tb = kTbCopy * wave + i;
      const uint32_t off = xl[u] + (uint32_t)(16 * tb + 4 * u) * (uint32_t)K * 2u + (uint32_t)kt * 256u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (__attribute__((address_space(3))) void*)(buf + tb * kXBlock + 1024 * u), 16, off, 0, 0, 0);
    }
}

// The A operand of k-step t of row block j: the tile's dword t widened and
// scaled by the k-step's group scale (G = 128 one per tile, the low or high
// half of the word of 2 tiles; G = 64 two; G = 32 four).
template <int GSH>
__device__ __forceinline__ half8_t w_widen1(const WTile<GSH>& T, int j, int t, int kt, uint32_t vmask,
                                            uint32_t vmask4, uint32_t vmagic) {
  half2_t sc;
  if constexpr (GSH == 0) sc = splat_sel_w(T.sraw[j][0], (kt & 1) ? kSelHiW : kSelLoW);
  else if constexpr (GSH == 1) sc = splat_sel_w(T.sraw[j][0], t < 2 ? kSelLoW : kSelHiW);
  else sc = splat_sel_w(T.sraw[j][t >> 1], (t & 1) ? kSelHiW : kSelLoW);
  const uint32_t w = t == 0 ? T.code[j].x : t == 1 ? T.code[j].y : t == 2 ? T.code[j].z : T.code[j].w;
  return dequant_dword(w, sc, vmask, vmask4, vmagic);
}

// One stage: the wave's 4 x 8 accumulator tiles over the code tile's 4
// k-steps of 32 columns. Per k-step the 8 token blocks' B operands are read
// from LDS first, then row block by row block its A operand is widened and
// its 8 MFMAs issue: the widening of the next row block runs among them (the
// two waves of a SIMD leave each barrier together, so widening in a block of
// its own would idle the matrix unit).
template <int GSH>
__device__ __forceinline__ void w_stage(float4_t (&acc)[kRbWave][kTbWave], const WTile<GSH>& T,
                                        const uint8_t* xw, const uint32_t (&xpos)[4], int kt, uint32_t vmask,
                                        uint32_t vmask4, uint32_t vmagic) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    half8_t b[kTbWave];
#pragma unroll
    for (int tb = 0; tb < kTbWave; ++tb) b[tb] = *reinterpret_cast<const half8_t*>(xw + tb * kXBlock + 16 * xpos[t]);
#pragma unroll
    for (int j = 0; j < kRbWave; ++j) {
      const half8_t a = w_widen1<GSH>(T, j, t, kt, vmask, vmask4, vmagic);
#pragma unroll
      for (int tb = 0; tb < kTbWave; ++tb) acc[j][tb] = mfma16(a, b[tb], acc[j][tb]);
    }
    __builtin_amdgcn_sched_barrier(0);   // one k-step's operands at a time
  }
}

template <int GSH>
__global__ __launch_bounds__(kThreadsW, 1) void k_gemm_rw(const uint4* __restrict__ tiles,
                                                          const uint16_t* __restrict__ scales, int64_t sstride,
                                                          const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                          int M, int N, int K, int Kt, int Nb, int NT, int T) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_rw[];
  uint8_t* const buf0 = lds_rw;
  uint8_t* const buf1 = lds_rw + kXStage;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wn = wave & 3, wm = wave >> 2;
  const int tile = xcd_tile(blockIdx.x, T);
  const int mt = tile / NT, nt = tile - mt * NT;
  const int rbw = nt * (kBNW / kRowsPerBlock) + kRbWave * wn;   // the wave's first row block
  const int m0 = mt * kBMW;

  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + (int64_t)m0 * K), 0, (int)(min(kBMW, M - m0) * K * 2), kBufferRaw);
  uint32_t xl[4], xpos[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    xl[u] = ((uint32_t)(lane >> 4) * (uint32_t)K + 8u * x_load_chunk(lane, u)) * 2u;
    xpos[u] = x_read_pos(lane, u);
  }
  uint32_t vmask = 0x000F000Fu, vmask4 = 0x00F000F0u, vmagic = 0x64006400u;
  asm volatile("" : "+v"(vmask), "+v"(vmask4), "+v"(vmagic));   // keep the constants in VGPRs for v_and_or_b32

  // The accumulators start from zeros the compiler cannot see through (with
  // a literal zero it has been seen to rematerialise only some components),
  // each its own, in the accumulation registers: the MFMAs then update them
  // in place.
  float4_t acc[kRbWave][kTbWave];
#pragma unroll
  for (int j = 0; j < kRbWave; ++j)
#pragma unroll
    for (int tb = 0; tb < kTbWave; ++tb) {
      acc[j][tb] = float4_t{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(acc[j][tb]));
    }

  // Stage kt computes from buffer kt % 2 while the copies and loads of stage
  // kt + 1 (the last tile again past the end: in bounds, never used) fill
  // the other; a wave's copies into LDS complete with its loads, then the
  // barrier publishes them and frees the buffer just read. One stage per
  // iteration, with no exit inside: the accumulators then stay in place.
  WSrc S;
  S.tiles = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(tiles), 0, 0x7fffffff, kBufferRaw);
  S.scales = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, 0x7fffffff, kBufferRaw);
  S.tl = 16u * (uint32_t)lane;
  S.sl = (uint32_t)(lane & 15) * (uint32_t)sstride * 2u;
  const int xwo = kTbWave * wm * kXBlock;   // the wave's token blocks in a stage buffer
  WTile<GSH> Tn;
  x_copy(buf0, xr, xl, K, 0, wave);
  w_load<GSH>(Tn, S, sstride, Kt, Nb, rbw, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < Kt; ++kt) {
    const WTile<GSH> Tc = Tn;
    const int k1 = min(kt + 1, Kt - 1);
    uint8_t* const cur = (kt & 1) ? buf1 : buf0;
    uint8_t* const nxt = (kt & 1) ? buf0 : buf1;
    x_copy(nxt, xr, xl, K, k1, wave);
    w_load<GSH>(Tn, S, sstride, Kt, Nb, rbw, k1);
    w_stage<GSH>(acc, Tc, cur + xwo, xpos, kt, vmask, vmask4, vmagic);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // Lane n + 16 g of tile (j, tb) holds D[4 g + i][n]: output features
  // 4 g + i of row block rbw + j, token 16 tb + n of the wave's tokens.
#pragma unroll
  for (int j = 0; j < kRbWave; ++j)
#pragma unroll
    for (int tb = 0; tb < kTbWave; ++tb) {
      const int m = m0 + 16 * (kTbWave * wm + tb) + (lane & 15);
      const int n0 = (rbw + j) * kRowsPerBlock + 4 * (lane >> 4);
      if (m < M && rbw + j < Nb && n0 < N) store4(Y + (int64_t)m * N + n0, acc[j][tb], N - n0, (N & 3) == 0);
    }
}

template <int GSH>
hipError_t launch_rw(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_rw<GSH>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsW);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int NT = (int)((p->Nb + (kBNW / kRowsPerBlock) - 1) / (kBNW / kRowsPerBlock));
  const int MT = (int)((M + kBMW - 1) / kBMW);
  const int T = NT * MT;
  k_gemm_rw<GSH><<<dim3((unsigned)T), dim3(kThreadsW), kLdsW, s>>>(
      reinterpret_cast<const uint4*>(p->tiles), p->scales, p->sstride, X, Y, (int)M, (int)p->N, (int)p->K,
      (int)p->Kt, (int)p->Nb, NT, T);
  return hipGetLastError();
}

}  // namespace

bool gemm_rw_takes(const mq_packed* p, int64_t M) {
  if (p->blocks || p->nnz > 0 || (p->K % kTileCols) != 0) return false;
  const int64_t NT = (p->Nb + (kBNW / kRowsPerBlock) - 1) / (kBNW / kRowsPerBlock);
  const int64_t MT = (M + kBMW - 1) / kBMW;
  return NT * MT >= 200;   // about one round of workgroups on 256 CUs
}

hipError_t launch_gemm_rw(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (p->G == 128) return launch_rw<0>(p, X, M, Y, s);
  if (p->G == 64) return launch_rw<1>(p, X, M, Y, s);
  return launch_rw<2>(p, X, M, Y, s);
}

}  // namespace mq
