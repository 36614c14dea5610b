// Decode kernel (M <= 64): Y = X (deq(Q_base) + deq(R))^T, fused.
//
// ZipperEngine (MosaicQuant explainer, Methodology section 3) runs the sparse
// residual inside the dense 4-bit GEMM kernel so activations are read once and
// no partial outputs are merged by a second kernel. This MI355X version:
//   * one workgroup of 8 waves per 16-row block; wave w streams an eighth of
//     the row block's 1 KiB code tiles, all of its loads issued up front;
//   * each lane widens its 16 B of codes to exact fp16 q in registers
//     (v_and_or_b32 with the fp16 1024.0 pattern, then one packed subtract),
//     which are the A operands of four 16x16x32 MFMA steps with X^T (tokens as
//     columns) as B; the group scale multiplies the fp32 MFMA result per output
//     row, so s*q never rounds to fp16;
//   * the row block's residual entries are dealt to the 8 waves in chunks of
//     32 (so column-clustered outliers do not pile onto one wave); a chunk is
//     one more MFMA whose A is one-hot by row carrying the fp16 residual
//     values and whose B gathers the matching X columns -- it lands in the
//     same fp32 accumulators as the base;
//   * the 8 partial 16 x M tiles are summed in LDS in a fixed order.
#include "kernel_common.h"
#include "mq_internal.h"
#include "gemv_group.h"

namespace mq {
namespace {

constexpr int kWaves = 8;
// X rows in LDS are kXPad halfs (16 B) longer than K: with a row stride that
// is a multiple of the 128-byte bank period, the 16 lanes of an MFMA B
// fragment (16 token rows, same columns) would hit the same banks.
constexpr int kXPad = 8;
constexpr size_t kXldsMaxBytes = 64 * 1024;   // X is staged in LDS when M * K * 2 fits
constexpr int kTpb = 4;   // code tiles per batch of one wave

// clamp(v) helper for token rows: rows >= M read row 0, their outputs are never stored
template <int MB>
__device__ __forceinline__ void token_rows(int M, int r, int (&mrow)[MB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) mrow[mb] = (mb * 16 + r < M) ? mb * 16 + r : 0;
}

// Scales of the 4 output rows (4g+i) of one tile: NS = 128/G groups per tile.
template <int NS>
struct TileScales {
  uint32_t lo[4];   // groups 0,1 (fp16 pairs)
  uint32_t hi[4];   // groups 2,3 (G = 32 only)
};

template <int NS>
__device__ __forceinline__ void load_scales(TileScales<NS>& S, const uint16_t* __restrict__ scales,
                                            const int (&srow)[4], const bool (&rowok)[4], int kt) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int si = srow[i] + kt * NS;
    if (NS == 1) {
      S.lo[i] = scales[si];
    } else if (NS == 2) {
      S.lo[i] = *reinterpret_cast<const uint32_t*>(scales + si);
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(scales + si);
      S.lo[i] = v.x;
      S.hi[i] = v.y;
    }
    if (!rowok[i]) S.lo[i] = 0u;
    if (NS == 4 && !rowok[i]) S.hi[i] = 0u;
  }
}

// One code tile: widen, 4 MFMA steps per token block, scale per output row.
template <int MB, int NS, bool XLDS, bool PAD>
__device__ __forceinline__ void tile_mma(float4_t (&acc)[MB], const uint4 code, const TileScales<NS>& S,
                                         const uint16_t* __restrict__ X, const uint16_t* xs, const int (&mrow)[MB],
                                         int K, int ldx, int kt, int g, uint32_t vmask, uint32_t vmask4,
                                         uint32_t vmagic) {
  constexpr int SPG = 4 / NS;   // MFMA k-steps per scale group
  half8_t a[4];
  a[0] = widen_q(code.x, vmask, vmask4, vmagic);
  a[1] = widen_q(code.y, vmask, vmask4, vmagic);
  a[2] = widen_q(code.z, vmask, vmask4, vmagic);
  a[3] = widen_q(code.w, vmask, vmask4, vmagic);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    half8_t bx[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int seg = kt * kTileCols + 32 * s4;
      if (PAD && seg >= K)   // padded 32-column segment (uniform branch)
        bx[s4] = as_half8(make_uint4(0u, 0u, 0u, 0u));
      else if (XLDS)
        bx[s4] = *reinterpret_cast<const half8_t*>(xs + mrow[mb] * ldx + seg + 8 * g);
      else
        bx[s4] = as_half8(*reinterpret_cast<const uint4*>(X + (int64_t)mrow[mb] * K + seg + 8 * g));
    }
#pragma unroll
    for (int grp = 0; grp < NS; ++grp) {
      float4_t tacc = mfma16(a[grp * SPG], bx[grp * SPG], float4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int s4 = grp * SPG + 1; s4 < (grp + 1) * SPG; ++s4) tacc = mfma16(a[s4], bx[s4], tacc);
      const int sh = 16 * (grp & 1);
      const uint32_t* w = (grp >= 2) ? S.hi : S.lo;
      acc[mb].x = fmaf(h_to_f((w[0] >> sh) & 0xFFFFu), tacc.x, acc[mb].x);
      acc[mb].y = fmaf(h_to_f((w[1] >> sh) & 0xFFFFu), tacc.y, acc[mb].y);
      acc[mb].z = fmaf(h_to_f((w[2] >> sh) & 0xFFFFu), tacc.z, acc[mb].z);
      acc[mb].w = fmaf(h_to_f((w[3] >> sh) & 0xFFFFu), tacc.w, acc[mb].w);
    }
  }
}

// Everything one code tile needs, loaded ahead of its use by the general
// decode loop: the lane's 16 bytes of codes, the scales of its 4 rows, and the
// X fragments of every token block (zero for padded 32-column segments). No
// value is touched after its load (rows past N read the last row's scales and
// feed outputs that are never stored), so the loads stay in flight until the
// tile is computed.
template <int MB, int NS>
struct TileIn {
  uint4 code;
  TileScales<NS> S;
  half8_t bx[MB][4];
};

template <int MB, int NS, bool XLDS>
__device__ __forceinline__ void load_tile_in(TileIn<MB, NS>& T, const uint4* __restrict__ tiles, int64_t tbase,
                                             const uint16_t* __restrict__ scales, const int (&srow)[4],
                                             const uint16_t* __restrict__ X, const uint16_t* xs,
                                             const int (&mrow)[MB], int K, int ldx, int kt, int lane, int g) {
  T.code = tiles[(tbase + kt) * 64 + lane];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int si = srow[i] + kt * NS;
    if (NS == 1) {
      T.S.lo[i] = scales[si];
    } else if (NS == 2) {
      T.S.lo[i] = *reinterpret_cast<const uint32_t*>(scales + si);
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(scales + si);
      T.S.lo[i] = v.x;
      T.S.hi[i] = v.y;
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int seg = kt * kTileCols + 32 * s4;
      if (seg >= K)   // padded 32-column segment (uniform branch)
        T.bx[mb][s4] = as_half8(make_uint4(0u, 0u, 0u, 0u));
      else if (XLDS)
        T.bx[mb][s4] = *reinterpret_cast<const half8_t*>(xs + mrow[mb] * ldx + seg + 8 * g);
      else
        T.bx[mb][s4] = as_half8(*reinterpret_cast<const uint4*>(X + (int64_t)mrow[mb] * K + seg + 8 * g));
    }
  }
}

// tile_mma on a prefetched tile
template <int MB, int NS>
__device__ __forceinline__ void tile_mma_in(float4_t (&acc)[MB], const TileIn<MB, NS>& T, uint32_t vmask,
                                            uint32_t vmask4, uint32_t vmagic) {
  constexpr int SPG = 4 / NS;
  half8_t a[4];
  a[0] = widen_q(T.code.x, vmask, vmask4, vmagic);
  a[1] = widen_q(T.code.y, vmask, vmask4, vmagic);
  a[2] = widen_q(T.code.z, vmask, vmask4, vmagic);
  a[3] = widen_q(T.code.w, vmask, vmask4, vmagic);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int grp = 0; grp < NS; ++grp) {
      float4_t tacc = mfma16(a[grp * SPG], T.bx[mb][grp * SPG], float4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int s4 = grp * SPG + 1; s4 < (grp + 1) * SPG; ++s4) tacc = mfma16(a[s4], T.bx[mb][s4], tacc);
      const int sh = 16 * (grp & 1);
      const uint32_t* w = (grp >= 2) ? T.S.hi : T.S.lo;
      acc[mb].x = fmaf(h_to_f((w[0] >> sh) & 0xFFFFu), tacc.x, acc[mb].x);
      acc[mb].y = fmaf(h_to_f((w[1] >> sh) & 0xFFFFu), tacc.y, acc[mb].y);
      acc[mb].z = fmaf(h_to_f((w[2] >> sh) & 0xFFFFu), tacc.z, acc[mb].z);
      acc[mb].w = fmaf(h_to_f((w[3] >> sh) & 0xFFFFu), tacc.w, acc[mb].w);
    }
  }
}

// One residual chunk of 32 entries (8 per lane): an MFMA whose A is one-hot
// by output row and carries the fp16 residual values, B the X columns the
// entries name. `first` is the stream index of the chunk's first entry
// (window bookkeeping when K > 4096); rtp = tile_ptr of the row block.
template <int MB, bool XLDS, bool MW>
__device__ __forceinline__ void res_chunk(float4_t (&acc)[MB], const uint4 v0, const uint4 v1, uint32_t first,
                                          const uint32_t* __restrict__ rtp, int nwin,
                                          const uint16_t* __restrict__ X, const uint16_t* xs, const int (&mrow)[MB],
                                          int K, int ldx, int r, int g) {
  const uint32_t e[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  int col[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) col[u] = (int)ent_col(e[u]);
  if (MW) {   // column window of each entry: count the window starts at or below its stream index
    const uint32_t idx = first + 8 * g;
    for (int w = 1; w < nwin; ++w) {
      const uint32_t ws = rtp[32 * w];   // one load per window, shared by the 8 entries
#pragma unroll
      for (int u = 0; u < 8; ++u) col[u] += (idx + u >= ws) ? kColWindow : 0;
    }
  }
  u32x4_t av;
#pragma unroll
  for (int u = 0; u < 8; u += 2) {
    const uint32_t lo = (ent_row(e[u]) == (uint32_t)r) ? ent_delta(e[u]) : 0u;
    const uint32_t hi = (ent_row(e[u + 1]) == (uint32_t)r) ? ent_delta(e[u + 1]) : 0u;
    av[u >> 1] = lo | (hi << 16);
  }
  const half8_t a = __builtin_bit_cast(half8_t, av);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    u32x4_t bv;
    // X in LDS: the token row's base as one LDS byte address, so a gather
    // address is one shift-add of the column (2 instructions, not the 3 the
    // compiler otherwise emits)
    typedef __attribute__((address_space(3))) const uint16_t lds_u16;
    const uint32_t xrow = (uint32_t)reinterpret_cast<uintptr_t>(reinterpret_cast<lds_u16*>(
                              reinterpret_cast<uintptr_t>(xs))) + 2u * (uint32_t)(mrow[mb] * ldx);
    auto gather = [&](uint32_t ent) __attribute__((always_inline)) {
      uint32_t a;
      asm("v_lshl_add_u32 %0, %1, 1, %2" : "=v"(a) : "v"(ent_col(ent)), "v"(xrow));
      return (uint32_t)*reinterpret_cast<lds_u16*>((uintptr_t)a);
    };
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      uint32_t lo, hi;
      if (XLDS && !MW) {
        lo = gather(e[u]);
        hi = gather(e[u + 1]);
      } else if (XLDS) {
        lo = xs[mrow[mb] * ldx + col[u]];
        hi = xs[mrow[mb] * ldx + col[u + 1]];
      } else {
        lo = X[mrow[mb] * K + col[u]];
        hi = X[mrow[mb] * K + col[u + 1]];
      }
      bv[u >> 1] = lo | (hi << 16);
    }
    acc[mb] = mfma16(a, __builtin_bit_cast(half8_t, bv), acc[mb]);
  }
}

// Chunks c0, c0 + KS, c0 + 2 KS, ... (< nch) of a row block's residual
// stream (chunk c starts at stream index E0 + 32 c), with the entries of
// RD chunks in flight: a dense residual gives a wave many chunks, and
// loading each only when the previous one is done would expose the memory
// latency once per chunk. Chunks past nch read the zero entries after the
// stream, which add nothing; the chunks are added in the same order as one
// at a time.
template <int MB, bool XLDS, bool MW, int KS>
__device__ __forceinline__ void res_rest(float4_t (&acc)[MB], const uint32_t* __restrict__ entries, uint32_t E0,
                                         uint32_t c0, uint32_t nch, int zero_off, const uint32_t* __restrict__ rtp,
                                         int nwin, const uint16_t* __restrict__ X, const uint16_t* xs,
                                         const int (&mrow)[MB], int K, int ldx, int r, int g) {
  if (c0 >= nch) return;   // the same in every lane
  constexpr int RD = MB >= 4 ? 2 : 4;   // four token blocks leave room for two
  uint4 e[RD][2];
#pragma unroll
  for (int k = 0; k < RD; ++k) {
    const uint32_t c = c0 + (uint32_t)(k * KS);
    const uint4* e4 = reinterpret_cast<const uint4*>((c < nch ? entries + E0 + kChunk * c : entries + zero_off) + 8 * g);
    e[k][0] = e4[0];
    e[k][1] = e4[1];
  }
  for (uint32_t c = c0; c < nch; c += RD * KS) {
#pragma unroll
    for (int k = 0; k < RD; ++k) {
      const uint32_t ck = c + (uint32_t)(k * KS);
      // zero chunks cost little with X in LDS; with X in global memory or
      // several windows they are skipped
      if ((XLDS && !MW) || ck < nch)
        res_chunk<MB, XLDS, MW>(acc, e[k][0], e[k][1], E0 + kChunk * ck, rtp, nwin, X, xs, mrow, K, ldx, r, g);
      const uint32_t cn = ck + (uint32_t)(RD * KS);
      const uint4* e4 =
          reinterpret_cast<const uint4*>((cn < nch ? entries + E0 + kChunk * cn : entries + zero_off) + 8 * g);
      e[k][0] = e4[0];
      e[k][1] = e4[1];
    }
  }
}

// Scales of rows 4g..4g+3 for TPW consecutive tiles when G = 128: one vector
// load per row (TPW fp16 values, 8- or 16-byte aligned).
template <int TPW>
__device__ __forceinline__ void load_scales_run(uint32_t (&w)[4][TPW / 2], const uint16_t* __restrict__ scales,
                                                const int (&srow)[4], const bool (&rowok)[4], int kt0) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t* p = scales + srow[i] + kt0;
    if (TPW == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[i][0] = rowok[i] ? v.x : 0u;
      w[i][1] = rowok[i] ? v.y : 0u;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      w[i][0] = rowok[i] ? v.x : 0u;
      w[i][1] = rowok[i] ? v.y : 0u;
      w[i][2] = rowok[i] ? v.z : 0u;
      w[i][3] = rowok[i] ? v.w : 0u;
    }
  }
}

// Block residual kept as 4-bit code tiles (handles from mq_pack_blocks):
// row block rb's residual tiles are blk[rt_ptr[rb] .. rt_ptr[rb + 1]), tile i
// holds codes in the base tile layout and one fp32 scale per row; slot
// `zero` is an all-zero tile. K = 4096 here, so the column tile is blk & 31.
struct DenseRes {
  const uint32_t* rt_ptr;
  const uint4* tiles;
  const float* scale;
  const int32_t* blk;
  uint32_t zero;
};

struct ResTile {
  uint4 code;
  float4_t sc;   // scales of rows 4 g .. 4 g + 3
  int kt;
};

__device__ __forceinline__ void load_res_tile(ResTile& T, const DenseRes& D, uint32_t i, int lane, int g) {
  T.code = D.tiles[(int64_t)i * 64 + lane];
  T.sc = *reinterpret_cast<const float4_t*>(D.scale + (int64_t)i * kRowsPerBlock + 4 * g);
  T.kt = D.blk[i] & 31;
}

// One residual tile, like a base tile of its own scale: the exact 4-bit codes
// times the tile's X columns (from LDS) on the MFMA path, scaled per row in fp32.
__device__ __forceinline__ void res_tile(float4_t (&acc)[1], const ResTile& T, const uint16_t* xs, int mrow, int ldx,
                                         int g, uint32_t vmask, uint32_t vmask4, uint32_t vmagic) {
  const uint16_t* xp = xs + mrow * ldx + T.kt * kTileCols + 8 * g;
  float4_t tacc = mfma16(widen_q(T.code.x, vmask, vmask4, vmagic), *reinterpret_cast<const half8_t*>(xp),
                         float4_t{0.f, 0.f, 0.f, 0.f});
  tacc = mfma16(widen_q(T.code.y, vmask, vmask4, vmagic), *reinterpret_cast<const half8_t*>(xp + 32), tacc);
  tacc = mfma16(widen_q(T.code.z, vmask, vmask4, vmagic), *reinterpret_cast<const half8_t*>(xp + 64), tacc);
  tacc = mfma16(widen_q(T.code.w, vmask, vmask4, vmagic), *reinterpret_cast<const half8_t*>(xp + 96), tacc);
  acc[0].x = fmaf(T.sc.x, tacc.x, acc[0].x);
  acc[0].y = fmaf(T.sc.y, tacc.y, acc[0].y);
  acc[0].z = fmaf(T.sc.z, tacc.z, acc[0].z);
  acc[0].w = fmaf(T.sc.w, tacc.w, acc[0].w);
}

// Fast decode kernel for K = 4096 and up to 4 tokens (XR = M rounded up to a
// power of two). One workgroup of 8 waves per 16-row block, 4 code tiles
// per wave. Memory counters retire in issue order, so the issue order is
// the consumption order:
//   1. the wave's own 512 columns of X (16 B per lane per token row), and
//      the scales of its tiles;
//   2. code tiles 0 and 1;
//   3. the row block's residual offsets (scalar loads: waiting for them
//      overlaps the tiles in flight), then the wave's first two residual
//      chunks (indices wave and wave + 8);
//   4. code tiles 2 and 3.
// The X slices are written to LDS and published by a barrier that waits
// for LDS traffic only, while the code tiles are still in flight. Tiles 0
// and 1 are computed first, then the residual chunks (their X columns come
// from LDS), then tiles 2 and 3, so the residual work overlaps the second
// half of the stream. Partial 16 x 1 tiles are summed in LDS in a fixed
// order.
// RS > 0 (handles whose densest row block has more than 16 chunks): the
// row block's chunks 16 .. 16 + RS - 1 are copied straight from global
// memory into LDS after the code tiles, 8 chunks (1 KiB) per load
// instruction, all in flight together; a row block far denser than the rest
// (outliers clustered in a few rows) then waits one memory latency for its
// residual instead of one per 4 chunks of each wave. The chunks are added in
// the same order either way. Such a launch also starts the row blocks of
// more than 16 chunks first: workgroups 0 .. n - 1 take the n row blocks the
// handle lists (up to 64, with their stream offsets), and workgroup n + rb
// takes row block rb unless that one is listed, in which case it ends at
// once. The list and a bitmask of the workgroups that end are kernel
// arguments indexed by the workgroup alone, so a workgroup learns its row
// block from argument loads issued together with the others.
constexpr int kRegChunks = 2 * kWaves;   // chunks of a row block held in registers by k_gemv_x
static_assert(kRegChunks == kDenseRbChunks, "the dense list names the row blocks that stage chunks");
constexpr int kDenseMaskWords = 256;     // bitmask of the workgroups that end at once: up to 8192 workgroups

struct DenseList {
  uint32_t n;                         // listed row blocks (0: one workgroup per row block, in order)
  uint32_t rb[kDenseListMax];         // ascending
  uint32_t e0[kDenseListMax];         // first stream entry of each
  uint32_t nch[kDenseListMax];        // chunks of each
  uint32_t mask[kDenseMaskWords];     // bit b: workgroup b ends at once (its row block is listed)
};

// One workgroup of k_gemv_x on row block rb. RS = 0: its stream offsets read
// from tile_ptr, chunks past the first 16 through registers. RS > 0 and LST:
// a row block from the dense list (le0, lnch: its stream), whose chunks past
// the first 16 are staged in LDS, requested first; the listed and the other
// row blocks take separate code paths of the kernel, so the plain one never
// waits on a staging load. RS > 0 and !LST (every row block dense, too many
// to list): the chunks are staged once the offsets have been read.
template <int GSH, int XR, bool DR, int RS, bool LST>
__device__ __forceinline__ void gemv_x_block(const uint4* __restrict__ tiles, const uint16_t* __restrict__ scales,
                                             int sstride, const uint32_t* __restrict__ tile_ptr,
                                             const uint32_t* __restrict__ entries, const uint16_t* __restrict__ X,
                                             uint16_t* __restrict__ Y, int M, int N, int zero_off, const DenseRes& D,
                                             uint16_t* xs, float4_t (*red)[64], uint8_t* stg, int rb, uint32_t le0,
                                             uint32_t lnch) {
  constexpr int KS = 8, TPW = 4, K = 4096, Kt = 32, NS = 1 << GSH, LDX = K + kXPad;
  static_assert(RS % (8 * KS) == 0 && (!DR || RS == 0), "staged chunks: whole load instructions per wave");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int kt0 = wave * TPW, c0 = kt0 * kTileCols, tbase = rb * Kt;
  int mrow[1];
  token_rows<1>(M, r, mrow);

  // 0. (RS: a listed row block) chunks kRegChunks .. kRegChunks + nstg - 1
  // into LDS, requested first: instruction i of the workgroup (issued by
  // wave i mod 8) carries chunks 8 i .. 8 i + 7, lane l's 16 bytes landing at
  // 16 l. The stream's zero pad covers the chunks read past the row block,
  // which are never used.
  uint32_t nstg = 0;
  auto stage = [&](uint32_t e0, uint32_t nch) __attribute__((always_inline)) {
    nstg = nch > (uint32_t)kRegChunks ? min(nch - (uint32_t)kRegChunks, (uint32_t)RS) : 0u;
    const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(entries), 0, (int)((zero_off + kEntryPad) * 4), kBufferRaw);
    const uint32_t ebase = (e0 + (uint32_t)(kChunk * kRegChunks)) * 4u + 16u * (uint32_t)lane;
    for (uint32_t i = (uint32_t)wave; 8 * i < nstg; i += KS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(er, (__attribute__((address_space(3))) void*)(stg + 1024 * i), 16,
                                               ebase + 1024u * i, 0, 0, 0);
  };
  if constexpr (RS > 0 && LST) stage(le0, lnch);

  // 1. X slice (rows >= M repeat row 0, never stored) and scales (raw: the
  // rows past N are zeroed at use, after the loads have been issued)
  const uint16_t* xsrc = X + c0 + 8 * lane;
  uint4 x0, x1, x2, x3;
  x0 = *reinterpret_cast<const uint4*>(xsrc);
  if constexpr (XR > 1) x1 = *reinterpret_cast<const uint4*>(xsrc + (1 < M ? K : 0));
  if constexpr (XR > 2) {
    x2 = *reinterpret_cast<const uint4*>(xsrc + (2 < M ? 2 * K : 0));
    x3 = *reinterpret_cast<const uint4*>(xsrc + (3 < M ? 3 * K : 0));
  }
  int srow[4];
  bool rowok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rb * kRowsPerBlock + 4 * g + i;
    rowok[i] = row < N;
    srow[i] = min(row, N - 1) * sstride;
  }
  // NS = 1: the 4 tiles' scales of a row are one 8-byte load; else per tile
  uint2 sraw[4][NS == 1 ? 1 : TPW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (NS == 1) {
      sraw[i][0] = *reinterpret_cast<const uint2*>(scales + srow[i] + kt0);
    } else {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const uint16_t* sp = scales + srow[i] + (kt0 + t) * NS;
        if constexpr (NS == 2) sraw[i][t] = make_uint2(*reinterpret_cast<const uint32_t*>(sp), 0u);
        else sraw[i][t] = *reinterpret_cast<const uint2*>(sp);
      }
    }
  }

  // 2. code tiles 0 and 1
  const uint4* tp = tiles + (tbase + kt0) * 64 + lane;
  uint4 code[TPW];
  code[0] = tp[0];
  code[1] = tp[64];
  __builtin_amdgcn_sched_barrier(0);   // keep the issue order (no instruction crosses)

  // 3. residual chunks wave and wave + 8: two aligned 16-byte loads per lane
  // each (row-block segments are whole 32-entry chunks); an index past the
  // row block reads the zero entries after the stream. DR: residual tiles
  // wave and wave + 8 of the row block instead (past its end: the zero tile).
  uint32_t E0 = 0, nchunks = 0;
  uint4 ent[2][2];
  uint32_t R0 = 0, nrt = 0;
  ResTile rt[2];
  if constexpr (DR) {
    R0 = D.rt_ptr[rb];
    nrt = D.rt_ptr[rb + 1] - R0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t c = (uint32_t)(wave + j * KS);
      load_res_tile(rt[j], D, c < nrt ? R0 + c : D.zero, lane, g);
    }
  } else {
    if constexpr (RS > 0 && LST) {   // its stream from the list
      E0 = le0;
      nchunks = lnch;
    } else {
      E0 = tile_ptr[tbase];
      nchunks = (tile_ptr[tbase + Kt] - E0) / (uint32_t)kChunk;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t c = (uint32_t)(wave + j * KS);
      const uint32_t* ep = (c < nchunks) ? entries + E0 + kChunk * c : entries + zero_off;
      const uint4* e4 = reinterpret_cast<const uint4*>(ep + 8 * g);
      ent[j][0] = e4[0];
      ent[j][1] = e4[1];
    }
  }

  // 4. code tiles 2 and 3
  __builtin_amdgcn_sched_barrier(0);
  code[2] = tp[128];
  code[3] = tp[192];
  if constexpr (RS > 0 && !LST) stage(E0, nchunks);

  // X slices into LDS, published with a wait on LDS traffic only
  uint16_t* xdst = xs + c0 + 8 * lane;
  *reinterpret_cast<uint4*>(xdst) = x0;
  if constexpr (XR > 1) *reinterpret_cast<uint4*>(xdst + LDX) = x1;
  if constexpr (XR > 2) {
    *reinterpret_cast<uint4*>(xdst + 2 * LDX) = x2;
    *reinterpret_cast<uint4*>(xdst + 3 * LDX) = x3;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  uint32_t vmask = 0x000F000Fu, vmask4 = 0x00F000F0u, vmagic = 0x64006400u;
  asm volatile("" : "+v"(vmask), "+v"(vmask4), "+v"(vmagic));   // keep the constants in VGPRs for v_and_or_b32
  float4_t acc[1] = {float4_t{0.f, 0.f, 0.f, 0.f}};
  auto tile = [&](int t) __attribute__((always_inline)) {
    TileScales<NS> S;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (NS == 1) {
        const uint32_t w = (t < 2) ? sraw[i][0].x : sraw[i][0].y;
        S.lo[i] = rowok[i] ? (w >> (16 * (t & 1))) & 0xFFFFu : 0u;
      } else {
        S.lo[i] = rowok[i] ? sraw[i][t].x : 0u;
        if constexpr (NS == 4) S.hi[i] = rowok[i] ? sraw[i][t].y : 0u;
      }
    }
    tile_mma<1, NS, true, false>(acc, code[t], S, X, xs, mrow, K, LDX, kt0 + t, g, vmask, vmask4, vmagic);
  };
  tile(0);
  tile(1);
  if constexpr (DR) {
    // residual tiles of this wave (the zero tile adds nothing: no branch)
    res_tile(acc, rt[0], xs, mrow[0], LDX, g, vmask, vmask4, vmagic);
    res_tile(acc, rt[1], xs, mrow[0], LDX, g, vmask, vmask4, vmagic);
    tile(2);
    tile(3);
    for (uint32_t c = (uint32_t)(wave + 2 * KS); c < nrt; c += KS) {
      ResTile t2;
      load_res_tile(t2, D, R0 + c, lane, g);
      res_tile(acc, t2, xs, mrow[0], LDX, g, vmask, vmask4, vmagic);
    }
  } else {
    // residual chunks of this wave; a chunk past the row block is skipped (the
    // empty use keeps its load ahead of the tiles instead of inside the branch)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t c = (uint32_t)(wave + j * KS);
      if (c < nchunks)
        res_chunk<1, true, false>(acc, ent[j][0], ent[j][1], E0 + kChunk * c, tile_ptr + tbase, 1, X, xs, mrow, K, LDX,
                                  r, g);
      else
        asm volatile("" ::"v"(ent[j][0].x), "v"(ent[j][1].x));
    }
    tile(2);
    tile(3);
    if constexpr (RS > 0) {
      if (nstg > 0) {   // the same in every wave of the workgroup
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // two chunks a round: both chunks' entries and X gathers are in
        // flight together, and the MFMAs keep the chunk order
        uint32_t c = (uint32_t)wave;
        for (; c + KS < nstg; c += 2 * KS) {
          const uint4* ep = reinterpret_cast<const uint4*>(stg + 128 * c + 32 * g);
          const uint4* eq = reinterpret_cast<const uint4*>(stg + 128 * (c + KS) + 32 * g);
          const uint4 a0 = ep[0], a1 = ep[1], b0 = eq[0], b1 = eq[1];
          res_chunk<1, true, false>(acc, a0, a1, 0u, tile_ptr + tbase, 1, X, xs, mrow, K, LDX, r, g);
          res_chunk<1, true, false>(acc, b0, b1, 0u, tile_ptr + tbase, 1, X, xs, mrow, K, LDX, r, g);
        }
        if (c < nstg) {
          const uint4* ep = reinterpret_cast<const uint4*>(stg + 128 * c + 32 * g);
          res_chunk<1, true, false>(acc, ep[0], ep[1], 0u, tile_ptr + tbase, 1, X, xs, mrow, K, LDX, r, g);
        }
      }
    }
    res_rest<1, true, false, KS>(acc, entries, E0, (uint32_t)(wave + kRegChunks + RS), nchunks, zero_off,
                                 tile_ptr + tbase, 1, X, xs, mrow, K, LDX, r, g);
  }

  red[wave][lane] = acc[0];
  __syncthreads();
  if (wave == 0) {
    float4_t sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < KS; ++w) sum += red[w][lane];
    const int n0 = rb * kRowsPerBlock + 4 * g;
    if (r < M) store4(Y + (int64_t)r * N + n0, sum, N - n0, (N & 3) == 0);
  }
}

template <int GSH, int XR, bool DR, int RS, bool LST>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(GSH == 0 ? 6 : GSH == 2 && RS > 0 ? 4 : 5, 8))) void k_gemv_x(
    const uint4* __restrict__ tiles, const uint16_t* __restrict__ scales, int sstride,
    const uint32_t* __restrict__ tile_ptr, const uint32_t* __restrict__ entries, const uint16_t* __restrict__ X,
    uint16_t* __restrict__ Y, int M, int N, int zero_off, DenseRes D, DenseList L) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [XR][4096 + kXPad]
  __shared__ float4_t red[kWaves][64];
  __shared__ __attribute__((aligned(16))) uint8_t stg[RS > 0 ? RS * kChunk * 4 : 16];   // staged chunks
  if constexpr (RS == 0 || !LST) {
    gemv_x_block<GSH, XR, DR, RS, false>(tiles, scales, sstride, tile_ptr, entries, X, Y, M, N, zero_off, D, xs, red,
                                         stg, (int)blockIdx.x, 0u, 0u);
  } else {
    // the list's fields at clamped indices, without branches, so that their
    // argument loads go out together
    const uint32_t b = blockIdx.x, bq = min(b, (uint32_t)kDenseListMax - 1);
    const uint32_t mw = L.mask[min(b >> 5, (uint32_t)kDenseMaskWords - 1)];
    const uint32_t lrb = L.rb[bq], le0 = L.e0[bq], lnch = L.nch[bq];
    if ((mw >> (b & 31)) & 1u) return;   // listed row block: taken by workgroup < n (the same in all waves)
    if (b < L.n)
      gemv_x_block<GSH, XR, false, RS, true>(tiles, scales, sstride, tile_ptr, entries, X, Y, M, N, zero_off, D, xs,
                                             red, stg, (int)lrb, le0, lnch);
    else
      gemv_x_block<GSH, XR, false, 0, false>(tiles, scales, sstride, tile_ptr, entries, X, Y, M, N, zero_off, D, xs,
                                             red, stg, (int)(b - L.n), 0u, 0u);
  }
}

// Decode kernel for K = 4096 and 5..16 tokens. X ([XR][4096] fp16, up to
// 128 KiB) fills most of the LDS, so one workgroup per CU holds it and works
// through R consecutive row blocks with it. X is copied in first (each wave
// its 512-column slice, straight from global memory into LDS) and published;
// then every wave requests the scales, its 4 code tiles and its first two
// residual chunks of all R row blocks before computing anything. The row
// blocks are computed in order (residual chunks gather their X columns from
// LDS) and the 8 partials of each are summed in LDS in a fixed order.
// The workgroup's body: row blocks rb0 .. rb0 + R - 1 of one layer.
template <int GSH, int XR, int R, bool DR>
__device__ __forceinline__ void gemv_r_block(const uint4* tiles, const uint16_t* scales, int sstride,
                                             const uint32_t* tile_ptr, const uint32_t* entries, const uint16_t* X,
                                             uint16_t* Y, int M, int N, int Nb, int zero_off, DenseRes D,
                                             const int rb0) {
  constexpr int KS = 8, TPW = 4, K = 4096, Kt = 32, NS = 1 << GSH, LDX = K + kXPad;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [XR][LDX], then the partials [R][KS][64]
  static_assert(R * KS * 64 * sizeof(float4_t) <= XR * LDX * sizeof(uint16_t), "partials fit in the X space");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int kt0 = wave * TPW, c0 = kt0 * kTileCols;
  int mrow[1];
  token_rows<1>(M, r, mrow);

  // residual segment of each row block (scalar loads, they land during the
  // X copy); DR: its residual tiles instead
  uint32_t E0[R], nch[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int rbc = min(rb0 + j, Nb - 1);
    if constexpr (DR) {
      E0[j] = D.rt_ptr[rbc];
      nch[j] = D.rt_ptr[rbc + 1] - E0[j];
    } else {
      const int tbase = rbc * Kt;
      E0[j] = tile_ptr[tbase];
      nch[j] = (tile_ptr[tbase + Kt] - E0[j]) / (uint32_t)kChunk;
    }
  }

  // X slice of this wave, one 1 KiB copy per token row straight from global
  // memory into LDS (rows >= M are never read), published before any code
  // tile is requested: X requests issued alongside the code stream queue
  // behind it in the memory system and would land only at its end.
#pragma unroll
  for (int m = 0; m < XR; ++m) {
    if (m < M)
      __builtin_amdgcn_global_load_lds(X + m * K + c0 + 8 * lane,
                                       (__attribute__((address_space(3))) void*)(xs + m * LDX + c0), 16, 0, 0);
  }
  __syncthreads();

  // everything the R row blocks need, requested before any of it is used,
  // row block by row block (scales, code tiles, the wave's first two
  // residual chunks: indices wave and wave + 8, zero entries past the end)
  uint4 code[R][TPW];
  uint2 sraw[R][4][NS == 1 ? 1 : TPW];
  uint4 ent[R][DR ? 1 : 2][2];
  ResTile rt[R];
  bool live[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int rb = min(rb0 + j, Nb - 1);   // a row block past the end repeats the last (never stored)
    live[j] = rb0 + j < Nb;
    const int tbase = rb * Kt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int srow = min(rb * kRowsPerBlock + 4 * g + i, N - 1) * sstride;
      if constexpr (NS == 1) {
        sraw[j][i][0] = *reinterpret_cast<const uint2*>(scales + srow + kt0);
      } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const uint16_t* sp = scales + srow + (kt0 + t) * NS;
          if constexpr (NS == 2) sraw[j][i][t] = make_uint2(*reinterpret_cast<const uint32_t*>(sp), 0u);
          else sraw[j][i][t] = *reinterpret_cast<const uint2*>(sp);
        }
      }
    }
    const uint4* tp = tiles + (tbase + kt0) * 64 + lane;
#pragma unroll
    for (int t = 0; t < TPW; ++t) code[j][t] = tp[t * 64];
    if constexpr (DR) {   // residual tile `wave` of the row block (past its end: the zero tile)
      const uint32_t c = (uint32_t)wave;
      load_res_tile(rt[j], D, c < nch[j] ? E0[j] + c : D.zero, lane, g);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t c = (uint32_t)(wave + h * KS);
        const uint32_t* ep = (c < nch[j]) ? entries + E0[j] + kChunk * c : entries + zero_off;
        const uint4* e4 = reinterpret_cast<const uint4*>(ep + 8 * g);
        ent[j][h][0] = e4[0];
        ent[j][h][1] = e4[1];
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // keep row block j's requests ahead of row block j + 1's
  }


  uint32_t vmask = 0x000F000Fu, vmask4 = 0x00F000F0u, vmagic = 0x64006400u;
  asm volatile("" : "+v"(vmask), "+v"(vmask4), "+v"(vmagic));   // keep the constants in VGPRs for v_and_or_b32
  float4_t part[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int rb = min(rb0 + j, Nb - 1);
    float4_t acc[1] = {float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      TileScales<NS> S;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rb * kRowsPerBlock + 4 * g + i < N;
        if constexpr (NS == 1) {
          const uint32_t w = (t < 2) ? sraw[j][i][0].x : sraw[j][i][0].y;
          S.lo[i] = ok ? (w >> (16 * (t & 1))) & 0xFFFFu : 0u;
        } else {
          S.lo[i] = ok ? sraw[j][i][t].x : 0u;
          if constexpr (NS == 4) S.hi[i] = ok ? sraw[j][i][t].y : 0u;
        }
      }
      tile_mma<1, NS, true, false>(acc, code[j][t], S, X, xs, mrow, K, LDX, kt0 + t, g, vmask, vmask4, vmagic);
    }
    if constexpr (DR) {   // residual tiles wave, wave + 8, ... (the zero tile adds nothing)
      res_tile(acc, rt[j], xs, mrow[0], LDX, g, vmask, vmask4, vmagic);
      for (uint32_t c = (uint32_t)(wave + KS); c < nch[j]; c += KS) {
        ResTile t2;
        load_res_tile(t2, D, E0[j] + c, lane, g);
        res_tile(acc, t2, xs, mrow[0], LDX, g, vmask, vmask4, vmagic);
      }
    } else {
      const uint32_t* rtp = tile_ptr + rb * Kt;
#pragma unroll
      for (int h = 0; h < 2; ++h) {   // a chunk past the row block is skipped; the empty use keeps its load in place
        if ((uint32_t)(wave + h * KS) < nch[j])
          res_chunk<1, true, false>(acc, ent[j][h][0], ent[j][h][1], E0[j] + kChunk * (wave + h * KS), rtp, 1, X, xs,
                                    mrow, K, LDX, r, g);
        else
          asm volatile("" ::"v"(ent[j][h][0].x), "v"(ent[j][h][1].x));
      }
      res_rest<1, true, false, KS>(acc, entries, E0[j], (uint32_t)(wave + 2 * KS), nch[j], zero_off, rtp, 1, X, xs,
                                   mrow, K, LDX, r, g);
    }
    part[j] = acc[0];
  }
  // the partials go where X was, once every wave is done with X
  float4_t* red = reinterpret_cast<float4_t*>(xs);   // [R][KS][64]
  __syncthreads();
#pragma unroll
  for (int j = 0; j < R; ++j) red[(j * KS + wave) * 64 + lane] = part[j];
  __syncthreads();
  if (wave < R && live[wave]) {   // wave j sums row block j
    const int j = wave, rb = rb0 + j;
    float4_t sum = red[(j * KS) * 64 + lane];
#pragma unroll
    for (int w = 1; w < KS; ++w) sum += red[(j * KS + w) * 64 + lane];
    const int n0 = rb * kRowsPerBlock + 4 * g;
    if (r < M) store4(Y + (int64_t)r * N + n0, sum, N - n0, (N & 3) == 0);
  }
}

template <int GSH, int XR, int R, bool DR>
__global__ __launch_bounds__(512) void k_gemv_r(const uint4* __restrict__ tiles, const uint16_t* __restrict__ scales,
                                               int sstride, const uint32_t* __restrict__ tile_ptr,
                                               const uint32_t* __restrict__ entries, const uint16_t* __restrict__ X,
                                               uint16_t* __restrict__ Y, int M, int N, int Nb, int zero_off,
                                               DenseRes D) {
  gemv_r_block<GSH, XR, R, DR>(tiles, scales, sstride, tile_ptr, entries, X, Y, M, N, Nb, zero_off, D,
                               blockIdx.x * R);
}

// Several layers of K = 4096 (element-wise or no residual, one group size)
// with inputs of the same token count in one launch: layer i owns
// workgroups wg0[i] .. wg0[i + 1] - 1, each of R of its row blocks, which
// are computed exactly as k_gemv_r computes them (the same sums in the same
// order), so each output equals that layer's own launch bit for bit. More
// row blocks per workgroup than one small layer can fill amortise the copy
// of X into LDS (at 16 tokens as many bytes per workgroup as 4 row blocks
// of codes), and the layers' ramps and tails overlap.
struct GroupR {
  const uint4* tiles[kGroupMax];
  const uint16_t* scales[kGroupMax];
  const uint32_t* tile_ptr[kGroupMax];
  const uint32_t* entries[kGroupMax];
  const uint16_t* X[kGroupMax];
  uint16_t* Y[kGroupMax];
  int sstride[kGroupMax], N[kGroupMax], Nb[kGroupMax], zero_off[kGroupMax];
  int wg0[kGroupMax + 1];   // first workgroup of each layer; wg0[n] = the grid
  int n;
};

template <int GSH, int XR, int R>
__global__ __launch_bounds__(512) void k_gemv_r_group(const GroupR G, int M) {
  const int b = (int)blockIdx.x;
  int li = 0;
#pragma unroll
  for (int i = 1; i < kGroupMax; ++i) li += (i < G.n && b >= G.wg0[i]) ? 1 : 0;
  li = __builtin_amdgcn_readfirstlane(li);
  const DenseRes none{nullptr, nullptr, nullptr, nullptr, 0u};
  gemv_r_block<GSH, XR, R, false>(G.tiles[li], G.scales[li], G.sstride[li], G.tile_ptr[li], G.entries[li], G.X[li],
                                  G.Y[li], M, G.N[li], G.Nb[li], G.zero_off[li], none, (b - G.wg0[li]) * R);
}

// The same for 1..4 tokens: k_gemv_x's body, one row block per workgroup
// (wg0[i] = the row blocks before layer i), with RS = 0 when every layer's
// densest row block holds at most kRegChunks residual chunks, else with the
// chunks past those staged in LDS, up to 64 (a row block of at most
// kRegChunks chunks stages none, and is computed as with RS = 0).
template <int GSH, int XR, int RS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(GSH == 0 ? 6 : GSH == 2 && RS > 0 ? 4 : 5, 8)))
void k_gemv_x_group(const GroupR G, int M) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [XR][4096 + kXPad]
  __shared__ float4_t red[kWaves][64];
  __shared__ __attribute__((aligned(16))) uint8_t stg[RS > 0 ? RS * kChunk * 4 : 16];   // staged chunks
  const int b = (int)blockIdx.x;
  int li = 0;
#pragma unroll
  for (int i = 1; i < kGroupMax; ++i) li += (i < G.n && b >= G.wg0[i]) ? 1 : 0;
  li = __builtin_amdgcn_readfirstlane(li);
  const DenseRes none{nullptr, nullptr, nullptr, nullptr, 0u};
  gemv_x_block<GSH, XR, false, RS, false>(G.tiles[li], G.scales[li], G.sstride[li], G.tile_ptr[li], G.entries[li],
                                          G.X[li], G.Y[li], M, G.N[li], G.zero_off[li], none, xs, red, stg,
                                          b - G.wg0[li], 0u, 0u);
}

// General decode kernel. KS waves per row block. GSH = log2(128 / G).
// XR > 0: X is copied whole into LDS ([M][K] within [XR][K]) and published
// before the code tiles are requested, else X fragments come from global
// memory. MW: K > 4096
// (several column windows). TPW > 0: every wave owns exactly TPW tiles
// (Kt == KS * TPW, K % 128 == 0) and issues all its loads up front; TPW == 0:
// any shape, one tile per iteration.
// Occupancy: all row blocks of a decode layer should be resident at once, so
// each SIMD must hold 6 waves of 8-wave groups (80 VGPRs).
template <int KS, int MB, int GSH, int XR, bool MW, int TPW>
__global__ __launch_bounds__(64 * KS) __attribute__((amdgpu_waves_per_eu(KS == 8 && TPW == 4 && MB == 1 && GSH == 0 ? 6 : 1, 8))) void k_gemv(const uint4* __restrict__ tiles,
                                                  const uint16_t* __restrict__ scales, int sstride,
                                                  const uint32_t* __restrict__ tile_ptr,
                                                  const uint32_t* __restrict__ entries,
                                                  const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                  int M, int N, int K, int Kt, int zero_off) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [M][LDX] when XR > 0
  constexpr bool XLDS = XR > 0;
  const int LDX = K + kXPad;
  __shared__ float4_t red[KS][MB][64];
  constexpr int NS = 1 << GSH;
  const int rb = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int kt0 = TPW ? wave * TPW : (Kt * wave) / KS;
  const int kt1 = TPW ? kt0 + TPW : (Kt * (wave + 1)) / KS;
  const int tbase = rb * Kt;
  int mrow[MB];
  token_rows<MB>(M, r, mrow);

  // ---- loads, in the order the tile loop consumes them (memory counters
  // retire in issue order, so whatever a tile needs is issued before the
  // code tiles it waits for).
  int srow[4];
  bool rowok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rb * kRowsPerBlock + 4 * g + i;
    rowok[i] = row < N;
    srow[i] = min(row, N - 1) * sstride;
  }
  constexpr int NT = TPW ? TPW : 1;
  constexpr bool RUN = TPW > 0 && NS == 1;   // G = 128: one vector load of scales per row
  uint32_t srun[4][RUN ? TPW / 2 : 1];
  TileScales<NS> S[NT];
  if constexpr (RUN) {
    load_scales_run<TPW>(srun, scales, srow, rowok, kt0);
  } else if (TPW) {
#pragma unroll
    for (int t = 0; t < NT; ++t) load_scales<NS>(S[t], scales, srow, rowok, kt0 + t);
  }

  if (XLDS) {   // whole X, straight from global memory into LDS (1 KiB per copy, by row), then published
    const int nck = (K + 511) >> 9;
    for (int idx = wave; idx < M * nck; idx += KS) {
      const int m = idx / nck, c = (idx - m * nck) * 512;
      if (c + 8 * lane < K)
        __builtin_amdgcn_global_load_lds(X + (int64_t)m * K + c + 8 * lane,
                                         (__attribute__((address_space(3))) void*)(xs + m * LDX + c), 16, 0, 0);
    }
    __syncthreads();
  }

  // ---- code tiles of the wave (fast path): all issued before anything waits
  uint4 code[NT];
  if (TPW) {
    const uint4* tp = tiles + (tbase + kt0) * 64 + lane;
#pragma unroll
    for (int t = 0; t < NT; ++t) code[t] = tp[t * 64];
  }

  // ---- the wave's first two residual chunks (indices wave and wave + KS),
  // requested ahead of the tile loop. Row-block segments of the stream are
  // whole 32-entry chunks (zero padded), so a chunk is two aligned 16-byte
  // loads per lane; a chunk index past the row block reads the zero entries
  // after the stream. Both are processed unconditionally after the tiles.
  const uint32_t E0 = tile_ptr[tbase], E1 = tile_ptr[tbase + Kt];
  const uint32_t nchunks = (E1 - E0) / (uint32_t)kChunk;
  const int nwin = (Kt + 31) >> 5;
  uint4 ent[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t c = (uint32_t)(wave + j * KS);
    const uint32_t* ep = (c < nchunks) ? entries + E0 + kChunk * c : entries + zero_off;
    const uint4* e4 = reinterpret_cast<const uint4*>(ep + 8 * g);
    ent[j][0] = e4[0];
    ent[j][1] = e4[1];
  }

  uint32_t vmask = 0x000F000Fu, vmask4 = 0x00F000F0u, vmagic = 0x64006400u;
  asm volatile("" : "+v"(vmask), "+v"(vmask4), "+v"(vmagic));   // keep the constants in VGPRs for v_and_or_b32

  float4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
  if (TPW) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (RUN) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t].lo[i] = (srun[i][t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
      }
      tile_mma<MB, NS, XLDS, false>(acc, code[t], S[t], X, xs, mrow, K, LDX, kt0 + t, g, vmask, vmask4, vmagic);
    }
  } else {
    // a ring of PDG register sets, each loaded PDG tiles ahead of its use;
    // the loop body takes PDG tiles and has no branch (a guarded refill would
    // make the compiler wait for the other sets' loads); the last tiles follow
    constexpr int PDG = MB == 1 ? 4 : MB == 2 ? 2 : 1;   // four token blocks: no room for a second set
    TileIn<MB, NS> T[PDG];
    const int last = Kt - 1;
#pragma unroll
    for (int u = 0; u < PDG; ++u)
      load_tile_in<MB, NS, XLDS>(T[u], tiles, tbase, scales, srow, X, xs, mrow, K, LDX, min(kt0 + u, last), lane, g);
    int kt = kt0;
    for (; kt + PDG <= kt1; kt += PDG) {
#pragma unroll
      for (int u = 0; u < PDG; ++u) {
        tile_mma_in<MB, NS>(acc, T[u], vmask, vmask4, vmagic);
        load_tile_in<MB, NS, XLDS>(T[u], tiles, tbase, scales, srow, X, xs, mrow, K, LDX, min(kt + PDG + u, last),
                                   lane, g);
      }
    }
#pragma unroll
    for (int u = 0; u < PDG - 1; ++u)
      if (kt + u < kt1) tile_mma_in<MB, NS>(acc, T[u], vmask, vmask4, vmagic);
  }

  // ---- residual: chunks wave, wave + KS, ... of the row block's entries
  res_chunk<MB, XLDS, MW>(acc, ent[0][0], ent[0][1], E0 + kChunk * wave, tile_ptr + tbase, nwin, X, xs, mrow, K, LDX, r, g);
  res_chunk<MB, XLDS, MW>(acc, ent[1][0], ent[1][1], E0 + kChunk * (wave + KS), tile_ptr + tbase, nwin, X, xs, mrow, K,
                          LDX, r, g);
  res_rest<MB, XLDS, MW, KS>(acc, entries, E0, (uint32_t)(wave + 2 * KS), nchunks, zero_off, tile_ptr + tbase, nwin, X,
                             xs, mrow, K, LDX, r, g);

  // ---- fixed-order sum of the KS partial tiles, fp16 output
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  if (wave < MB) {
    const int mb = wave;
    float4_t s = red[0][mb][lane];
#pragma unroll
    for (int w = 1; w < KS; ++w) s += red[w][mb][lane];
    const int m = mb * 16 + r;                   // token
    const int n0 = rb * kRowsPerBlock + 4 * g;   // first of 4 output features
    if (m < M) store4(Y + (int64_t)m * N + n0, s, N - n0, (N & 3) == 0);
  }
}

constexpr size_t kXldsMax = kXldsMaxBytes;

// once per kernel instantiation: allow kXldsMax bytes of dynamic LDS
template <typename F>
hipError_t allow_lds(F* fn, bool& done) {
  if (done) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)kXldsMax);
  if (e == hipSuccess) done = true;
  return e;
}

// the block residual of a handle from mq_pack_blocks as code tiles (unused otherwise)
DenseRes dense_res(const mq_packed* p) {
  return DenseRes{p->rt_ptr, reinterpret_cast<const uint4*>(p->rt_tiles), p->bscale, p->blk, (uint32_t)p->nblk};
}

constexpr size_t kLdsMaxBytes = 160 * 1024;   // LDS of one CU

// the handle's dense row blocks for a launch that takes them first
DenseList dense_list(const mq_packed* p) {
  DenseList L{};
  if (p->ndense <= (uint32_t)kDenseListMax && p->Nb + p->ndense <= 32 * kDenseMaskWords) {
    L.n = p->ndense;
    for (uint32_t i = 0; i < L.n; ++i) {
      L.rb[i] = p->dense_rb[i];
      L.e0[i] = p->dense_e0[i];
      L.nch[i] = p->dense_nch[i];
      const uint32_t b = L.n + L.rb[i];   // the workgroup that would take it in order
      L.mask[b >> 5] |= 1u << (b & 31);
    }
  }
  return L;
}

// LST: the handle's dense row blocks go first, one workgroup more per listed
// row block (whose in-order workgroup ends at once)
template <int GSH, int XR, bool DR, int RS, bool LST>
hipError_t launch_x(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  // dynamic LDS: X (the partials and the staged chunks are static)
  constexpr size_t lds = (size_t)XR * (4096 + kXPad) * 2;
  static bool done = false;
  if (!done) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_x<GSH, XR, DR, RS, LST>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    done = true;
  }
  const DenseList L = LST ? dense_list(p) : DenseList{};
  k_gemv_x<GSH, XR, DR, RS, LST><<<dim3((unsigned)(p->Nb + L.n)), dim3(512), lds, s>>>(
      reinterpret_cast<const uint4*>(p->tiles), p->scales, (int)p->sstride, p->tile_ptr, p->entries, X, Y, M,
      (int)p->N, (int)p->stream_cap, dense_res(p), L);
  return hipGetLastError();
}

// Element-wise residual: LDS staging sized to the densest row block
// (beyond 16 + 256 chunks the rest goes through registers as below 16),
// the dense row blocks first when the handle lists them.
template <int GSH, int XR>
hipError_t launch_x_res(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  const uint32_t mc = p->max_rb / (uint32_t)kChunk;
  if (mc <= (uint32_t)kRegChunks) return launch_x<GSH, XR, false, 0, false>(p, X, M, Y, s);
  const bool lst = dense_list(p).n > 0;
  if (mc <= (uint32_t)kRegChunks + 64)
    return lst ? launch_x<GSH, XR, false, 64, true>(p, X, M, Y, s) : launch_x<GSH, XR, false, 64, false>(p, X, M, Y, s);
  return lst ? launch_x<GSH, XR, false, 256, true>(p, X, M, Y, s) : launch_x<GSH, XR, false, 256, false>(p, X, M, Y, s);
}

// Row blocks per workgroup of the K = 4096 decode body over layers of nb[i]
// row blocks. X fills the LDS, so the workgroups run in rounds of one per
// CU, and a workgroup of R row blocks takes about R + 0.64 row-block times
// (0.64 for its copy of X): on the six K = 4096 layers of a 4096-hidden
// block at 16 tokens (2400 row blocks), 2 / 4 / 5 row blocks per workgroup
// in 5 / 3 / 2 rounds took 34.9 / 36.5 / 30.7 us. The pick is the R with the
// least rounds x (R + 0.64) up to rmax, the most that fit the registers
// without spills (5 for G = 128, 4 for G = 64, 2 for G = 32).
int rows_per_workgroup(const int* nb, int n, int rmax) {
  int best_r = 1;
  double best = 1e300;
  for (int R = 1; R <= rmax; ++R) {
    int wg = 0;
    for (int i = 0; i < n; ++i) wg += (nb[i] + R - 1) / R;
    const double cost = (double)((wg + 255) / 256) * (R + 0.64);
    if (cost < best) {
      best = cost;
      best_r = R;
    }
  }
  return best_r;
}

template <int GSH, int XR, int R, bool DR>
hipError_t launch_r(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  static bool done = false;
  if (!done) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_r<GSH, XR, R, DR>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMaxBytes);
    if (e != hipSuccess) return e;
    done = true;
  }
  const unsigned grid = (unsigned)((p->Nb + R - 1) / R);
  k_gemv_r<GSH, XR, R, DR><<<dim3(grid), dim3(512), (size_t)XR * (4096 + kXPad) * 2, s>>>(
      reinterpret_cast<const uint4*>(p->tiles), p->scales, (int)p->sstride, p->tile_ptr, p->entries, X, Y, M,
      (int)p->N, (int)p->Nb, (int)p->stream_cap, dense_res(p));
  return hipGetLastError();
}

// Row blocks per workgroup: X fills the LDS, so one workgroup runs per CU,
// and ceil(Nb / 256) row blocks each make one round of workgroups (a few
// workgroups past 256 would take a second round on their own). Up to 4 row
// blocks fit the registers, 2 when G = 32 (4 scales per tile and row); past
// one round of 4 (layers of more than 16384 rows) the rounds model of
// rows_per_workgroup picks, with 5 for G = 128 (block residuals keep 4).
template <int GSH, int XR, bool DR>
hipError_t launch_r_any(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  if (p->Nb <= 256) return launch_r<GSH, XR, 1, DR>(p, X, M, Y, s);
  if constexpr (GSH == 2) {
    return launch_r<GSH, XR, 2, DR>(p, X, M, Y, s);
  } else {
    if (p->Nb <= 512) return launch_r<GSH, XR, 2, DR>(p, X, M, Y, s);
    if (p->Nb <= 768) return launch_r<GSH, XR, 3, DR>(p, X, M, Y, s);
    if constexpr (!DR) {
      if (p->Nb > 1024) {
        const int nb = (int)p->Nb;
        switch (rows_per_workgroup(&nb, 1, GSH == 0 ? 5 : 4)) {
          case 1: return launch_r<GSH, XR, 1, DR>(p, X, M, Y, s);
          case 2: return launch_r<GSH, XR, 2, DR>(p, X, M, Y, s);
          case 3: return launch_r<GSH, XR, 3, DR>(p, X, M, Y, s);
          case 5:
            if constexpr (GSH == 0) return launch_r<GSH, XR, 5, DR>(p, X, M, Y, s);
            break;
        }
      }
    }
    return launch_r<GSH, XR, 4, DR>(p, X, M, Y, s);
  }
}

template <int GSH, int XR, int R>
hipError_t launch_r_group(const GroupR& G, int grid, int M, hipStream_t s) {
  static bool done = false;
  if (!done) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_r_group<GSH, XR, R>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMaxBytes);
    if (e != hipSuccess) return e;
    done = true;
  }
  k_gemv_r_group<GSH, XR, R><<<dim3((unsigned)grid), dim3(512), (size_t)XR * (4096 + kXPad) * 2, s>>>(G, M);
  return hipGetLastError();
}

template <int GSH, int XR>
hipError_t launch_r_group_any(GroupR& G, int M, hipStream_t s) {
  constexpr int kRmax = GSH == 0 ? 5 : GSH == 1 ? 4 : 2;
  const int R = rows_per_workgroup(G.Nb, G.n, kRmax);
  int wg = 0;
  for (int i = 0; i < G.n; ++i) {
    G.wg0[i] = wg;
    wg += (G.Nb[i] + R - 1) / R;
  }
  for (int i = G.n; i <= kGroupMax; ++i) G.wg0[i] = wg;
  switch (R) {
    case 1: return launch_r_group<GSH, XR, 1>(G, wg, M, s);
    case 2: return launch_r_group<GSH, XR, 2>(G, wg, M, s);
  }
  if constexpr (kRmax >= 4) {
    if (R == 3) return launch_r_group<GSH, XR, 3>(G, wg, M, s);
    if (R == 4) return launch_r_group<GSH, XR, 4>(G, wg, M, s);
  }
  if constexpr (kRmax >= 5) {
    if (R == 5) return launch_r_group<GSH, XR, 5>(G, wg, M, s);
  }
  return hipErrorInvalidValue;
}

template <int GSH, int XR, int RS>
hipError_t launch_x_group(GroupR& G, int M, hipStream_t s) {
  constexpr size_t lds = (size_t)XR * (4096 + kXPad) * 2;
  static bool done = false;
  if (!done) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_x_group<GSH, XR, RS>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    done = true;
  }
  int wg = 0;
  for (int i = 0; i < G.n; ++i) {
    G.wg0[i] = wg;
    wg += G.Nb[i];
  }
  for (int i = G.n; i <= kGroupMax; ++i) G.wg0[i] = wg;
  k_gemv_x_group<GSH, XR, RS><<<dim3((unsigned)wg), dim3(512), lds, s>>>(G, M);
  return hipGetLastError();
}

template <int GSH, int XR>
hipError_t launch_x_group_rs(GroupR& G, int M, bool staged, hipStream_t s) {
  return staged ? launch_x_group<GSH, XR, 64>(G, M, s) : launch_x_group<GSH, XR, 0>(G, M, s);
}

template <int GSH>
hipError_t launch_group_g(GroupR& G, int M, bool staged, hipStream_t s) {
  if (M == 1) return launch_x_group_rs<GSH, 1>(G, M, staged, s);
  if (M == 2) return launch_x_group_rs<GSH, 2>(G, M, staged, s);
  if (M <= 4) return launch_x_group_rs<GSH, 4>(G, M, staged, s);
  return M <= 8 ? launch_r_group_any<GSH, 8>(G, M, s) : launch_r_group_any<GSH, 16>(G, M, s);
}

// XL: X copied whole into LDS ([M][K + kXPad], at most kXldsMax bytes)
template <int KS, int MB, int GSH, int XL, bool MWV, int TPW>
hipError_t launch(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  if (XL) {
    static bool done = false;
    const hipError_t e = allow_lds(&k_gemv<KS, MB, GSH, XL, MWV, TPW>, done);
    if (e != hipSuccess) return e;
  }
  k_gemv<KS, MB, GSH, XL, MWV, TPW><<<dim3((unsigned)p->Nb), dim3(64 * KS), XL ? (size_t)M * (p->K + kXPad) * 2 : 0,
                                      s>>>(
      reinterpret_cast<const uint4*>(p->tiles), p->scales, (int)p->sstride, p->tile_ptr, p->entries, X, Y, M,
      (int)p->N, (int)p->K, (int)p->Kt, (int)p->stream_cap);
  return hipGetLastError();
}

// Waves per row block and tiles per wave: the fast path needs Kt = KS * TPW;
// 8 waves x 4 tiles when Kt = 32 (K = 4096), 4 x 4 for K = 2048, 8 x 8 for
// K = 8192 (one token block only: more would not fit the registers), else
// the generic one-tile loop over 8 waves.
template <int MB, int GSH, int XL, bool MWV>
hipError_t pick_shape(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  const bool k128 = (p->K % kTileCols) == 0;
  if constexpr (!MWV) {
    if (k128 && p->Kt == 32) return launch<kWaves, MB, GSH, XL, false, 4>(p, X, M, Y, s);
    if (k128 && p->Kt == 16) return launch<4, MB, GSH, XL, false, 4>(p, X, M, Y, s);
  } else if constexpr (MB == 1) {
    if (k128 && p->Kt == 64) return launch<kWaves, MB, GSH, XL, true, 8>(p, X, M, Y, s);
  }
  return launch<kWaves, MB, GSH, XL, MWV, 0>(p, X, M, Y, s);
}

template <int MB, int GSH, int XL>
hipError_t run_x(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  return p->Kt > 32 ? pick_shape<MB, GSH, XL, true>(p, X, M, Y, s) : pick_shape<MB, GSH, XL, false>(p, X, M, Y, s);
}

template <int MB, int GSH>
hipError_t run(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  if constexpr (MB == 1) {
    if (p->K == 4096 && M <= 4) {   // fast kernel: X slices in LDS, residual amid the tiles
      if (p->blocks) {   // the block residual as code tiles
        if (M == 1) return launch_x<GSH, 1, true, 0, false>(p, X, M, Y, s);
        if (M == 2) return launch_x<GSH, 2, true, 0, false>(p, X, M, Y, s);
        return launch_x<GSH, 4, true, 0, false>(p, X, M, Y, s);
      }
      if (M == 1) return launch_x_res<GSH, 1>(p, X, M, Y, s);
      if (M == 2) return launch_x_res<GSH, 2>(p, X, M, Y, s);
      return launch_x_res<GSH, 4>(p, X, M, Y, s);
    }
    if (p->K == 4096) {   // 5..16 tokens: X whole in LDS, several row blocks per workgroup
      if (p->blocks) {
        if (M <= 8) return launch_r_any<GSH, 8, true>(p, X, M, Y, s);
        return launch_r_any<GSH, 16, true>(p, X, M, Y, s);
      }
      if (M <= 8) return launch_r_any<GSH, 8, false>(p, X, M, Y, s);
      return launch_r_any<GSH, 16, false>(p, X, M, Y, s);
    }
    if ((size_t)M * (p->K + kXPad) * 2 <= kXldsMax) return run_x<MB, GSH, 1>(p, X, M, Y, s);
  }
  return run_x<MB, GSH, 0>(p, X, M, Y, s);
}

template <int MB>
hipError_t run_g(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  if (p->G == 128) return run<MB, 0>(p, X, M, Y, s);
  if (p->G == 64) return run<MB, 1>(p, X, M, Y, s);
  return run<MB, 2>(p, X, M, Y, s);
}

}  // namespace

bool gemv_group_takes(const mq_packed* const* p, int n, int64_t M) {
  if (n < 1 || n > kGroupMax || M < 1 || M > 16) return false;
  for (int i = 0; i < n; ++i) {
    if (p[i]->K != 4096 || p[i]->blocks || p[i]->G != p[0]->G || p[i]->device != p[0]->device) return false;
    // up to 4 tokens, row blocks of at most kRegChunks + 64 residual chunks
    // (the kernel variants of launch_x_res without the overflow loop)
    if (M <= 4 && p[i]->max_rb / (uint32_t)kChunk > (uint32_t)kRegChunks + 64) return false;
  }
  return true;
}

hipError_t launch_gemv_group(const mq_packed* const* p, const uint16_t* const* X, int64_t M, uint16_t* const* Y,
                             int n, hipStream_t s) {
  if (!gemv_group_takes(p, n, M)) return hipErrorInvalidValue;
  GroupR G{};
  G.n = n;
  for (int i = 0; i < n; ++i) {
    G.tiles[i] = reinterpret_cast<const uint4*>(p[i]->tiles);
    G.scales[i] = p[i]->scales;
    G.tile_ptr[i] = p[i]->tile_ptr;
    G.entries[i] = p[i]->entries;
    G.X[i] = X[i];
    G.Y[i] = Y[i];
    G.sstride[i] = (int)p[i]->sstride;
    G.N[i] = (int)p[i]->N;
    G.Nb[i] = (int)p[i]->Nb;
    G.zero_off[i] = (int)p[i]->stream_cap;
  }
  bool staged = false;   // up to 4 tokens: some row block holds more than kRegChunks chunks
  for (int i = 0; i < n; ++i) staged |= p[i]->max_rb / (uint32_t)kChunk > (uint32_t)kRegChunks;
  if (p[0]->G == 128) return launch_group_g<0>(G, (int)M, staged, s);
  if (p[0]->G == 64) return launch_group_g<1>(G, (int)M, staged, s);
  return launch_group_g<2>(G, (int)M, staged, s);
}

hipError_t launch_gemv(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  // Block-residual handles carry their residual as code tiles only, which
  // the K = 4096 kernels up to 16 tokens multiply; otherwise the mid-size
  // kernel (any K, up to 64 tokens) takes them.
  if (p->blocks && (p->K != 4096 || M > 16)) return launch_gemm_mid(p, X, M, Y, s);
  if (M <= 16) return run_g<1>(p, X, (int)M, Y, s);
  if (M <= 32) return run_g<2>(p, X, (int)M, Y, s);
  return run_g<4>(p, X, (int)M, Y, s);
}

}  // namespace mq
