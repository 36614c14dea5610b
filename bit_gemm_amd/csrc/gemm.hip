// Prefill kernel (any M): Y = X (deq(Q_base) + deq(R))^T, fused.
//
// ZipperEngine (MosaicQuant explainer, Methodology section 3) runs the sparse
// residual inside the dense 4-bit GEMM so X is read once and no partial
// outputs are merged afterwards. Here the residual is folded into the dense
// weight tile before the matrix cores consume it:
//   * a workgroup of 8 waves computes a 256 (output features) x 256 (tokens)
//     tile, each wave a 128 x 64 block of 4 x 2 32x32x16 fp16 MFMAs with
//     fp32 accumulators (two waves per SIMD); up to 128 tokens a 256 x 64
//     tile of 8 waves of 32 x 64 (Cfg); when the tiles cannot fill the GPU,
//     K is split across workgroups and a second kernel adds the fp32 parts;
//   * K advances in stages of 64 columns (half a code tile), double-buffered
//     in LDS: the weight stage is widened from the 4-bit tiles to fp16(s q)
//     by the wave that owns those 2 row blocks, which then patches the
//     stage's residual entries into it (fp16(s q + sr qr), rounded once) --
//     a wave's LDS operations execute in order, so no barrier is needed
//     between its writes and its patches; X is staged through registers;
//   * one loop iteration is one code tile (two stages; four with the
//     narrow tile's ring); its body has no branches, so the widening,
//     patching and X staging of the next stage interleave with the current
//     stage's MFMAs; one barrier per stage;
//   * workgroups are ordered so that consecutive tiles of one 256-token
//     slice run on the same XCD and share its L2 for X.
// Handles from mq_pack_blocks (Methodology section 2: residual blocks) carry
// their residual as 4-bit code tiles; for them (DR) each stage also widens
// the tile's residual codes with the row's residual scale and adds them to
// the staged weights, instead of patching single entries.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "kernel_common.h"
#include "mq_internal.h"

namespace mq {
namespace {

typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int BN = 256;               // output features per workgroup (16 row blocks)
constexpr int BK = 64;                // K columns per LDS stage
constexpr int LDW = BK + 8;           // LDS row (halves): 144 B, so 8 consecutive rows hit distinct banks
constexpr int kSplitTarget = 256;       // workgroups to aim for when K is split (one per CU)

// Workgroup shape: a BN x BM_ output tile (features x tokens) computed by
// NWN_ x NWM_ waves, each owning a (BN / NWN_) x (BM_ / NWM_) block of 32x32
// MFMA tiles.
//   * Wide (BM 256, 2 x 4 waves of 128 x 64): 128 accumulators per wave, two
//     waves per SIMD, so one wave's stalls are covered by the other's MFMAs.
//   * Narrow (BM 64, 8 x 1 waves of 32 x 64), for up to a few dozen tokens:
//     a wide tile would spend three quarters of its MFMAs on token rows past
//     M; here every wave still widens two of the 16 row blocks. Its stages
//     are short and its accumulators few, so the loads run four stages
//     ahead (a ring of register sets) instead of two, which keeps twice as
//     many bytes in flight to cover the memory latency.
template <int BM_, int NWN_, int NWM_, int PD_>
struct Cfg {
  static constexpr int kBM = BM_;
  static constexpr int kNwn = NWN_, kNwm = NWM_;
  static constexpr int kWaves = NWN_ * NWM_;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRb = 16 / kWaves;              // row blocks widened and patched by each wave
  static constexpr int kIb = BN / NWN_ / 32;           // 32-feature MFMA blocks per wave
  static constexpr int kJb = BM_ / NWM_ / 32;          // 32-token MFMA blocks per wave
  static constexpr int kXr = BM_ * BK / 8 / kThreads;  // 16-byte X chunks per thread per stage
  static constexpr int kPd = PD_;                      // stages loaded ahead: 2, or a ring of 4 or 8
  static constexpr size_t kStageHalves = (size_t)(BN + BM_) * LDW;
  static constexpr size_t kDummyOff = 2 * kStageHalves * sizeof(_Float16);   // [64] halves: patch targets of idle lanes
  static constexpr size_t kLdsBytes = kDummyOff + 64 * sizeof(_Float16);
  static_assert(kWaves * kRb == 16 && kXr >= 1 && kIb >= 1 && kJb >= 1, "workgroup shape");
};
using CfgWide = Cfg<256, 2, 4, 2>;
using CfgNarrow = Cfg<64, 8, 1, 4>;
#ifndef MQ_GEMM_NARROW_MAX_M
#define MQ_GEMM_NARROW_MAX_M 128
#endif
constexpr int64_t kNarrowMaxM = MQ_GEMM_NARROW_MAX_M;   // token counts up to this use the narrow shape

// Widened weights are stored as this type: it may alias anything, so the
// compiler keeps the patches' atomic XORs on the same LDS words after them.
typedef uint32_t lds_u32x4_t __attribute__((ext_vector_type(4), __may_alias__));

// XOR v into the 16-bit LDS element `half` of the stage buffer (an atomic on
// its dword: two patches may share one)
__device__ __forceinline__ void xor_half(_Float16* Ws, uint32_t half, uint32_t v) {
  (void)__hip_atomic_fetch_xor(reinterpret_cast<uint32_t*>(Ws) + (half >> 1), v << (16 * (half & 1u)),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// v_perm_b32 selectors: the low / high fp16 of a dword in both halves
constexpr uint32_t kSelLo = 0x05040100u, kSelHi = 0x07060302u;
__device__ __forceinline__ half2_t splat_sel(uint32_t dword, uint32_t sel) {
  return __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dword, dword, sel));
}

// Residual segment bounds of one code tile for the wave's RB row blocks
// (wave-uniform, so they live in scalar registers). They are fetched a full
// iteration before the entry loads that use them as addresses.
template <int RB>
struct TilePtrs {
  uint32_t p0[RB], cnt[RB];
};

// Block residual kept as 4-bit code tiles (handles from mq_pack_blocks):
// slot[rb * Kt + kt] is the residual tile of (rb, kt), or an all-zero slot;
// tiles in the base tile layout, one fp32 scale per row.
struct DenseGemm {
  const int32_t* slot;
  const uint2* tiles;
  const float* scale;
};

// DR: p0 holds the residual slot of the tile (no patched-weight entries).
template <bool DR, int RB>
__device__ __forceinline__ void load_ptrs(TilePtrs<RB>& P, const uint32_t* __restrict__ tile_ptr,
                                          const DenseGemm& dr, int Kt, int Nb, int rbw, int kt) {
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const bool ok = rbw + j < Nb && kt < Kt;
    const int64_t t = (int64_t)min(rbw + j, Nb - 1) * Kt + min(kt, Kt - 1);
    if constexpr (DR) {
      P.p0[j] = (uint32_t)dr.slot[t];
      P.cnt[j] = 0u;
    } else {
      const uint32_t p0 = tile_ptr[t], p1 = tile_ptr[t + 1];
      P.p0[j] = p0;
      P.cnt[j] = ok ? p1 - p0 : 0u;
    }
  }
}

// Registers holding one half (64 columns, one LDS stage) of a code tile for
// the wave's RB row blocks. Each half set is refilled in place right after
// its last use, two stages ahead of the next one, so the loop never copies
// registers that are still being loaded (a copy would wait for the load).
// Nothing is selected at load time either (a select waits for its load):
// row blocks past the layer and tiles past K are clamped to the last ones
// and only feed output rows that are never stored or stages that are never
// run; rows past N inside a row block have scale 0.
template <int RB>
struct HalfRegs {
  uint2 code[RB];        // dwords 2h, 2h + 1 of the lane's 16-byte slice of the tile
  uint32_t sraw[RB];     // the aligned dword of the lane's scale row holding this stage's scale(s)
  uint32_t sel;          // byte selector of the scale in it (G = 128 / 64; scalar)
  uint32_t ent[RB];      // patched-weight entry p0 + lane of the tile's segment (valid when lane < cnt);
                         // DR: fp32 bits of the residual scale of the lane's row
  uint32_t cnt[RB];      // entries in the tile's segment (scalar)
  uint2 rcode[RB];       // DR: the same two dwords of the tile's residual codes
};

template <int RB>
__device__ __forceinline__ bool has_long_segment(const HalfRegs<RB>& H) {
  bool any = false;
#pragma unroll
  for (int j = 0; j < RB; ++j) any = any || H.cnt[j] > 64;
  return any;
}

// Branch- and wait-free: clamped indices keep every load in bounds (1024 zero
// entries follow the stream, so p0 + lane is always readable).
template <int GSH, bool DR, int RB>
__device__ __forceinline__ void load_half(HalfRegs<RB>& H, const TilePtrs<RB>& P, const uint4* __restrict__ tiles,
                                          const uint16_t* __restrict__ scales, int64_t sstride,
                                          const uint32_t* __restrict__ wpatch, const DenseGemm& dr, int Kt, int Nb,
                                          int rbw, int kt, int h, int lane) {
  const int r = lane & 15;
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int rb = min(rbw + j, Nb - 1), ktc = min(kt, Kt - 1);
    const int64_t t = (int64_t)rb * Kt + ktc;
    H.code[j] = reinterpret_cast<const uint2*>(tiles)[(t * 64 + lane) * 2 + h];
    const uint16_t* srow = scales + (int64_t)(rb * kRowsPerBlock + r) * sstride;
    // whole aligned dwords (scale rows are padded to 8 halves): a 16-bit load
    // would need a zero-extension, which the compiler may place right after
    // the load and so wait for it a stage early
    if constexpr (GSH == 0) H.sraw[j] = reinterpret_cast<const uint32_t*>(srow)[ktc >> 1];
    else if constexpr (GSH == 1) H.sraw[j] = reinterpret_cast<const uint32_t*>(srow)[ktc];
    else H.sraw[j] = *reinterpret_cast<const uint32_t*>(srow + 4 * ktc + 2 * h);
    if constexpr (DR) {
      H.rcode[j] = dr.tiles[((int64_t)P.p0[j] * 64 + lane) * 2 + h];
      H.ent[j] = __builtin_bit_cast(uint32_t, dr.scale[(int64_t)P.p0[j] * kRowsPerBlock + r]);
    } else {
      H.ent[j] = wpatch[P.p0[j] + lane];
    }
    H.cnt[j] = P.cnt[j];
  }
  H.sel = (GSH == 0 ? (min(kt, Kt - 1) & 1) : h) ? kSelHi : kSelLo;
}

// X stage [BM tokens][BK columns]: XR x 16 B per thread, 8 consecutive chunks of
// a row per 8 lanes; thread tid reads rows tid / 8 + (THREADS / 8) i, chunk
// tid % 8. The
// loads go through a buffer resource over the workgroup's rows of X (base row
// m0, `nrec` = valid rows x K x 2 bytes): rows past M read as zero by the
// hardware's range check, so one offset register serves all 8 rows and no
// load needs a guard (a guarded load would become a branch). Columns past K
// (a K tail, or the look-ahead past the last stage) read the next row or
// zero; with a K tail they are masked to zero with a mask kept opaque to the
// compiler (a select would be turned back into a branch), otherwise they
// land in a stage that is never consumed.
template <bool KTAIL, int XR, int THREADS>
__device__ __forceinline__ void load_x(uint4 (&x)[XR], __amdgpu_buffer_rsrc_t xrs, uint32_t xoff, int K, int col0,
                                       int tid) {
  uint32_t keep = col0 + 8 * (tid & 7) < K ? ~0u : 0u;
  if (KTAIL) asm volatile("" : "+v"(keep));
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const uint32_t off = xoff + (uint32_t)((THREADS / 8) * i * K + col0) * 2u;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
    x[i] = KTAIL ? make_uint4(v[0] & keep, v[1] & keep, v[2] & keep, v[3] & keep) : make_uint4(v[0], v[1], v[2], v[3]);
  }
}

template <int XR, int THREADS>
__device__ __forceinline__ void store_x(const uint4 (&x)[XR], _Float16* Xs, int tid) {
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int idx = tid + THREADS * i;
    *reinterpret_cast<uint4*>(Xs + (idx >> 3) * LDW + 8 * (idx & 7)) = x[i];
  }
}

// Widen half h of the tile (dwords 2h, 2h + 1) of the wave's row blocks to
// fp16(s q) in the stage buffer, then overwrite the positions of the first
// 64 residual entries of each tile segment that fall in this half with their
// patched weights. A wave's LDS writes execute in order, so a patch lands
// after the widened value it replaces; no other wave writes these rows.
// Lanes without an entry write to their own dummy slot. The target offset is
// blended with a mask hidden behind an empty asm: written as a select, it
// becomes an exec-masked branch, and branches split the stage into separate
// scheduling regions, which keeps the widening from interleaving with the
// MFMAs.
// DR: the residual tile's codes are widened the same way with the row's
// residual scale (rounded to fp16) and added in fp16; no patches follow.
template <int GSH, bool DR, int RB>
__device__ __forceinline__ void write_w(const HalfRegs<RB>& H, _Float16* Ws, _Float16* dummy, int lrb0, int h,
                                        int lane, uint32_t vmask, uint32_t vmask4, uint32_t vmagic) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    _Float16* dst = Ws + ((lrb0 + j) * kRowsPerBlock + r) * LDW + 8 * g;
    const half2_t s0 = splat_sel(H.sraw[j], GSH == 2 ? kSelLo : H.sel);
    const half2_t s1 = GSH == 2 ? splat_sel(H.sraw[j], kSelHi) : s0;
    half8_t w0 = dequant_dword(H.code[j].x, s0, vmask, vmask4, vmagic);
    half8_t w1 = dequant_dword(H.code[j].y, s1, vmask, vmask4, vmagic);
    if constexpr (DR) {
      const _Float16 sr = (_Float16)__builtin_bit_cast(float, H.ent[j]);
      const half2_t srs = {sr, sr};
      w0 += dequant_dword(H.rcode[j].x, srs, vmask, vmask4, vmagic);
      w1 += dequant_dword(H.rcode[j].y, srs, vmask, vmask4, vmagic);
    }
    *reinterpret_cast<lds_u32x4_t*>(dst) = __builtin_bit_cast(lds_u32x4_t, w0);
    *reinterpret_cast<lds_u32x4_t*>(dst + 32) = __builtin_bit_cast(lds_u32x4_t, w1);
  }
  if constexpr (DR) return;
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const uint32_t v = H.ent[j];
    uint32_t okm = 0u - (((uint32_t)lane < H.cnt[j]) & ((v & kPatchValid) != 0u) & (((v >> 6) & 1u) == (uint32_t)h));
    asm("" : "+v"(okm));
    // both offsets are positive: the dummy slots follow the two stage buffers
    const uint32_t real = (uint32_t)(((lrb0 + j) * kRowsPerBlock + (int)ent_row(v)) * LDW) + (v & 63u);
    const uint32_t idle = (uint32_t)(dummy - Ws) + (uint32_t)lane;
    xor_half(Ws, idle ^ ((real ^ idle) & okm), v >> 16);
  }
}

// Entries 64.. of tile segments longer than 64 (dense residual tiles): rare,
// so the segment bounds are read again here instead of being kept in
// registers for every stage.
template <int RB>
__device__ __forceinline__ void patch_rest(const uint32_t* __restrict__ tile_ptr, int Kt, int Nb, int rbw, int kt,
                                           _Float16* Ws, int lrb0, int h, int lane,
                                           const uint32_t* __restrict__ wpatch) {
  TilePtrs<RB> P;
  load_ptrs<false>(P, tile_ptr, DenseGemm{}, Kt, Nb, rbw, kt);
  for (int j = 0; j < RB; ++j) {
    for (uint32_t e = P.p0[j] + 64 + lane; e < P.p0[j] + P.cnt[j]; e += 64) {
      const uint32_t v = wpatch[e];
      if ((v & kPatchValid) == 0u || ((v >> 6) & 1u) != (uint32_t)h) continue;
      const int row = (lrb0 + j) * kRowsPerBlock + (int)ent_row(v);
      xor_half(Ws, (uint32_t)(row * LDW) + (v & 63u), v >> 16);
    }
  }
}

// One stage of MFMAs: wave (wn, wm) multiplies its 32 IB weight rows by its
// 32 JB token columns over the stage's 64 columns (4 k-steps of 16). Lane l
// feeds row / column l % 32 and k 8 (l / 32) .. +7 of each 32x32x16 step.
template <int IB, int JB>
__device__ __forceinline__ void mfma_stage(float16_t (&acc)[IB][JB], const _Float16* Ws, const _Float16* Xs, int wn,
                                           int wm, int lane) {
  const int r32 = lane & 31, kh = 8 * (lane >> 5);
  const _Float16* wa = Ws + (32 * IB * wn + r32) * LDW + kh;
  const _Float16* xb = Xs + (32 * JB * wm + r32) * LDW + kh;
  half8_t a[2][IB], b[2][JB];
#pragma unroll
  for (int i = 0; i < IB; ++i) a[0][i] = *reinterpret_cast<const half8_t*>(wa + 32 * i * LDW);
#pragma unroll
  for (int j = 0; j < JB; ++j) b[0][j] = *reinterpret_cast<const half8_t*>(xb + 32 * j * LDW);
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int cb = ks & 1, nb = cb ^ 1;
    if (ks + 1 < BK / 16) {
#pragma unroll
      for (int i = 0; i < IB; ++i) a[nb][i] = *reinterpret_cast<const half8_t*>(wa + 32 * i * LDW + 16 * (ks + 1));
#pragma unroll
      for (int j = 0; j < JB; ++j) b[nb][j] = *reinterpret_cast<const half8_t*>(xb + 32 * j * LDW + 16 * (ks + 1));
    }
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[cb][i], b[cb][j], acc[i][j], 0, 0, 0);
  }
}

template <int GSH, bool KTAIL, class C, bool DR>
__global__ __launch_bounds__(C::kThreads, 1) void k_gemm(const uint4* __restrict__ tiles,
                                                      const uint16_t* __restrict__ scales, int64_t sstride,
                                                      const uint32_t* __restrict__ tile_ptr,
                                                      const uint32_t* __restrict__ wpatch,
                                                      const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                      float* __restrict__ part, int M, int N, int K, int Kt, int Nb,
                                                      int NT, int T, int kt_per_split, DenseGemm dr) {
  extern __shared__ __attribute__((aligned(16))) _Float16 lds[];
  constexpr int BM = C::kBM;
  _Float16* const dummy = reinterpret_cast<_Float16*>(reinterpret_cast<char*>(lds) + C::kDummyOff);
  _Float16* const buf0 = lds;
  _Float16* const buf1 = lds + C::kStageHalves;

  const int tile = xcd_tile(blockIdx.x, T);
  // split-K: this workgroup covers code tiles [kt0, kt1) (the whole K unless
  // the layer has too few output tiles to fill the chip)
  const int kt0 = blockIdx.y * kt_per_split, kt1 = min(Kt, kt0 + kt_per_split);
  const int mt = tile / NT, nt = tile - mt * NT;
  const int rb0 = nt * (BN / kRowsPerBlock), m0 = mt * BM;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, tid = threadIdx.x;
  constexpr int RB = C::kRb, IB = C::kIb, JB = C::kJb, XR = C::kXr, TH = C::kThreads;
  const int wn = wave % C::kNwn, wm = wave / C::kNwn;   // feature slice, token slice
  const int lrb0 = RB * wave;                // local row blocks widened by this wave
  const int rbw = rb0 + lrb0;
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + (int64_t)m0 * K), 0, (int)(min(BM, M - m0) * K * 2), kBufferRaw);
  const uint32_t xoff = (uint32_t)((tid >> 3) * K + 8 * (tid & 7)) * 2u;
  uint32_t vmask = 0x000F000Fu, vmask4 = 0x00F000F0u, vmagic = 0x64006400u;
  asm volatile("" : "+v"(vmask), "+v"(vmask4), "+v"(vmagic));   // keep the constants in VGPRs for v_and_or_b32

  float16_t acc[IB][JB];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Stage s = 2 kt + h is half h of tile kt. H0 / H1 hold the next even /
  // odd stage to prepare; pa / pb the segment bounds of the next refill of
  // H1 / H0.
  HalfRegs<RB> H0, H1;
  TilePtrs<RB> pa, pb;
  if constexpr (C::kPd == 2) {
  uint4 xr[XR];
  load_ptrs<DR>(pa, tile_ptr, dr, Kt, Nb, rbw, kt0);
  load_half<GSH, DR>(H0, pa, tiles, scales, sstride, wpatch, dr, Kt, Nb, rbw, kt0, 0, lane);
  load_half<GSH, DR>(H1, pa, tiles, scales, sstride, wpatch, dr, Kt, Nb, rbw, kt0, 1, lane);
  load_x<KTAIL, XR, TH>(xr, xrs, xoff, K, 2 * kt0 * BK, tid);
  write_w<GSH, DR>(H0, buf0, dummy, lrb0, 0, lane, vmask, vmask4, vmagic);
  if (has_long_segment(H0)) patch_rest<RB>(tile_ptr, Kt, Nb, rbw, kt0, buf0, lrb0, 0, lane, wpatch);
  store_x<XR, TH>(xr, buf0 + BN * LDW, tid);
  load_x<KTAIL, XR, TH>(xr, xrs, xoff, K, (2 * kt0 + 1) * BK, tid);
  load_ptrs<DR>(pa, tile_ptr, dr, Kt, Nb, rbw, kt0 + 1);
  load_half<GSH, DR>(H0, pa, tiles, scales, sstride, wpatch, dr, Kt, Nb, rbw, kt0 + 1, 0, lane);
  load_ptrs<DR>(pb, tile_ptr, dr, Kt, Nb, rbw, kt0 + 2);
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    // stage 2 kt (buffer 0) runs; stage 2 kt + 1 (H1: half 1 of tile kt) is prepared in buffer 1
    mfma_stage(acc, buf0, buf0 + BN * LDW, wn, wm, lane);
    write_w<GSH, DR>(H1, buf1, dummy, lrb0, 1, lane, vmask, vmask4, vmagic);
    store_x<XR, TH>(xr, buf1 + BN * LDW, tid);
    load_x<KTAIL, XR, TH>(xr, xrs, xoff, K, (2 * kt + 2) * BK, tid);
    const bool long1 = has_long_segment(H1);
    load_half<GSH, DR>(H1, pa, tiles, scales, sstride, wpatch, dr, Kt, Nb, rbw, kt + 1, 1, lane);
    load_ptrs<DR>(pa, tile_ptr, dr, Kt, Nb, rbw, kt + 2);
    if (long1) patch_rest<RB>(tile_ptr, Kt, Nb, rbw, kt, buf1, lrb0, 1, lane, wpatch);
    __syncthreads();
    // stage 2 kt + 1 (buffer 1) runs; stage 2 kt + 2 (H0: half 0 of tile kt + 1) is prepared in buffer 0
    mfma_stage(acc, buf1, buf1 + BN * LDW, wn, wm, lane);
    write_w<GSH, DR>(H0, buf0, dummy, lrb0, 0, lane, vmask, vmask4, vmagic);
    store_x<XR, TH>(xr, buf0 + BN * LDW, tid);
    load_x<KTAIL, XR, TH>(xr, xrs, xoff, K, (2 * kt + 3) * BK, tid);
    const bool long0 = has_long_segment(H0);
    load_half<GSH, DR>(H0, pb, tiles, scales, sstride, wpatch, dr, Kt, Nb, rbw, kt + 2, 0, lane);
    load_ptrs<DR>(pb, tile_ptr, dr, Kt, Nb, rbw, kt + 3);
    if (long0) patch_rest<RB>(tile_ptr, Kt, Nb, rbw, kt + 1, buf0, lrb0, 0, lane, wpatch);
    __syncthreads();
  }
  } else {
    // Ring of PD register sets: before stage s runs, set (s - sb + 1 + i) % PD
    // holds stage s + 1 + i (i < PD), all in flight. Stage s prepares stage
    // s + 1 from its set and refills that set with stage s + 1 + PD. PD is a
    // multiple of 4, so within the unrolled body every set index, tile half
    // and segment-bounds slot is a constant. The two slots of segment bounds
    // hold the tiles of even / odd index (from kt0); a slot is reloaded, two
    // tiles ahead, right after its tile's second half was requested.
    constexpr int PD = C::kPd;
    static_assert(PD == 4 || PD == 8, "ring depth");
    const int sb = 2 * kt0, se = 2 * kt1;   // the split's stages
    HalfRegs<RB> H[PD];
    TilePtrs<RB> Pr[2];
    uint4 xq[PD][XR];
    load_ptrs<DR>(Pr[0], tile_ptr, dr, Kt, Nb, rbw, kt0);
    load_ptrs<DR>(Pr[1], tile_ptr, dr, Kt, Nb, rbw, kt0 + 1);
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      load_x<KTAIL, XR, TH>(xq[u], xrs, xoff, K, (sb + u) * BK, tid);
      load_half<GSH, DR>(H[u], Pr[(u >> 1) & 1], tiles, scales, sstride, wpatch, dr, Kt, Nb, rbw, kt0 + (u >> 1),
                         u & 1, lane);
      if (u & 1) load_ptrs<DR>(Pr[(u >> 1) & 1], tile_ptr, dr, Kt, Nb, rbw, kt0 + (u >> 1) + 2);
    }
    write_w<GSH, DR>(H[0], buf0, dummy, lrb0, 0, lane, vmask, vmask4, vmagic);
    if (has_long_segment(H[0])) patch_rest<RB>(tile_ptr, Kt, Nb, rbw, kt0, buf0, lrb0, 0, lane, wpatch);
    store_x<XR, TH>(xq[0], buf0 + BN * LDW, tid);
    load_x<KTAIL, XR, TH>(xq[0], xrs, xoff, K, (sb + PD) * BK, tid);
    load_half<GSH, DR>(H[0], Pr[(PD >> 1) & 1], tiles, scales, sstride, wpatch, dr, Kt, Nb, rbw, kt0 + PD / 2, 0,
                       lane);
    __syncthreads();

    // stage s of the ring (U = (s - sb) % PD, a constant)
    auto stage = [&](auto uc, int s) {
      constexpr int u = decltype(uc)::value;
      _Float16* const cur = (u & 1) ? buf1 : buf0;
      _Float16* const nxt = (u & 1) ? buf0 : buf1;
      constexpr int v = (u + 1) % PD, h = (u + 1) & 1, pr = ((u + 1 + PD) >> 1) & 1;
      const int kl = kt0 + ((s + 1 + PD - sb) >> 1);   // tile of the stage requested now
      mfma_stage(acc, cur, cur + BN * LDW, wn, wm, lane);
      write_w<GSH, DR>(H[v], nxt, dummy, lrb0, h, lane, vmask, vmask4, vmagic);
      store_x<XR, TH>(xq[v], nxt + BN * LDW, tid);
      load_x<KTAIL, XR, TH>(xq[v], xrs, xoff, K, (s + 1 + PD) * BK, tid);
      const bool lng = has_long_segment(H[v]);
      load_half<GSH, DR>(H[v], Pr[pr], tiles, scales, sstride, wpatch, dr, Kt, Nb, rbw, kl, h, lane);
      if (h) load_ptrs<DR>(Pr[pr], tile_ptr, dr, Kt, Nb, rbw, kl + 2);
      if (lng) patch_rest<RB>(tile_ptr, Kt, Nb, rbw, kt0 + ((s + 1 - sb) >> 1), nxt, lrb0, h, lane, wpatch);
      __syncthreads();
    };
    // Whole turns of the ring run unguarded: a guard would let the compiler
    // assume a path on which the later stages' loads were not issued and wait
    // for the loads of the ring's next set too early.
    int s0 = sb;
    for (; s0 + PD <= se; s0 += PD) {
      stage(std::integral_constant<int, 0>{}, s0);
      stage(std::integral_constant<int, 1>{}, s0 + 1);
      stage(std::integral_constant<int, 2>{}, s0 + 2);
      stage(std::integral_constant<int, 3>{}, s0 + 3);
      if constexpr (PD == 8) {
        stage(std::integral_constant<int, 4>{}, s0 + 4);
        stage(std::integral_constant<int, 5>{}, s0 + 5);
        stage(std::integral_constant<int, 6>{}, s0 + 6);
        stage(std::integral_constant<int, 7>{}, s0 + 7);
      }
    }
    // the rest (fewer than PD stages; the same in every wave)
    if (s0 < se) stage(std::integral_constant<int, 0>{}, s0);
    if (s0 + 1 < se) stage(std::integral_constant<int, 1>{}, s0 + 1);
    if (s0 + 2 < se) stage(std::integral_constant<int, 2>{}, s0 + 2);
    if constexpr (PD == 8) {
      if (s0 + 3 < se) stage(std::integral_constant<int, 3>{}, s0 + 3);
      if (s0 + 4 < se) stage(std::integral_constant<int, 4>{}, s0 + 4);
      if (s0 + 5 < se) stage(std::integral_constant<int, 5>{}, s0 + 5);
      if (s0 + 6 < se) stage(std::integral_constant<int, 6>{}, s0 + 6);
    }
  }

  // Epilogue: register v of lane l holds D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32]
  // of each 32x32 block (rows = output features, columns = tokens). With
  // split-K the fp32 sums go to this split's slice of the workspace.
  const int nbase = rb0 * kRowsPerBlock + 32 * IB * wn + 4 * (lane >> 5);
  const int mbase = m0 + 32 * JB * wm + (lane & 31);
  float* const pslice = part ? part + (int64_t)blockIdx.y * M * N : nullptr;
#pragma unroll
  for (int i = 0; i < IB; ++i) {
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int m = mbase + 32 * j;
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n0 = nbase + 32 * i + 8 * q;
        if (n0 >= N) continue;
        const float4_t s = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if (pslice) {
          float* dst = pslice + (int64_t)m * N + n0;
          if ((N & 3) == 0 && n0 + 4 <= N) {
            *reinterpret_cast<float4_t*>(dst) = s;
          } else {
            for (int c = 0; c < 4 && n0 + c < N; ++c) dst[c] = s[c];
          }
        } else {
          store4(Y + (int64_t)m * N + n0, s, N - n0, (N & 3) == 0);
        }
      }
    }
  }
}

// Split-K reduction: Y = fp16(sum of the S partial slices), the slices added
// in split order (deterministic). One thread per 4 outputs of a token row;
// the slices are read 8 at a time so the loads overlap.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, uint16_t* __restrict__ Y,
                                                       int M, int N, int S) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;   // quad index
  const int nq = (N + 3) / 4;
  if (q >= (int64_t)M * nq) return;
  const int m = (int)(q / nq), n0 = 4 * (int)(q - (int64_t)m * nq);
  const int64_t slice = (int64_t)M * N;
  const float* src = part + (int64_t)m * N + n0;
  float4_t sum = {0.f, 0.f, 0.f, 0.f};
  if ((N & 3) == 0) {
    int sp = 0;
    for (; sp + 8 <= S; sp += 8) {
      float4_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4_t*>(src + (sp + u) * slice);
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; sp < S; ++sp) sum += *reinterpret_cast<const float4_t*>(src + sp * slice);
  } else {
    const int w = min(4, N - n0);
    for (int sp = 0; sp < S; ++sp)
      for (int c = 0; c < w; ++c) sum[c] += src[sp * slice + c];
  }
  store4(Y + (int64_t)m * N + n0, sum, N - n0, (N & 3) == 0);
}

// Workspace of the entry point that allocates nothing (mq_linear_noalloc):
// the split-K partial sums live in this array instead of a stream-ordered
// allocation. Host code never names it directly: its device address comes
// from hipGetSymbolAddress, once per device (each GPU has its own copy).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// split-K parts for a layer and token count (1 = no split)
template <class C>
int split_parts(const mq_packed* p, int64_t M, int* per_out) {
  const int NT = (int)((p->Nb + (BN / kRowsPerBlock) - 1) / (BN / kRowsPerBlock));
  const int MT = (int)((M + C::kBM - 1) / C::kBM);
  const int T = NT * MT;
  const int Kt = (int)p->Kt;
  // Split K when the output tiles cannot fill the chip's 256 CUs: about one
  // round of workgroups, at least 2 code tiles per split.
  int S = 1;
  if (T < kSplitTarget) S = std::max(1, std::min(kSplitTarget / T, Kt / 2));
  const int per = (Kt + S - 1) / S;
  if (per_out) *per_out = per;
  return (Kt + per - 1) / per;
}

// ws: caller's workspace for the split-K partials (nullptr: allocate it on
// the stream for this call)
template <int GSH, bool KTAIL, class C, bool DR>
hipError_t launch(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s, float* ws) {
  constexpr int BM = C::kBM;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<GSH, KTAIL, C, DR>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int NT = (int)((p->Nb + (BN / kRowsPerBlock) - 1) / (BN / kRowsPerBlock));
  const int MT = (int)((M + BM - 1) / BM);
  const int T = NT * MT;
  const int Kt = (int)p->Kt;
  int per = Kt;
  const int S = split_parts<C>(p, M, &per);
  float* part = nullptr;
  if (S > 1) {
    if (ws) {
      part = ws;
    } else {
      const hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&part), (size_t)S * M * p->N * sizeof(float), s);
      if (e != hipSuccess) return e;
    }
  }
  const DenseGemm dr = DR ? DenseGemm{p->rt_slot, reinterpret_cast<const uint2*>(p->rt_tiles), p->bscale}
                          : DenseGemm{nullptr, nullptr, nullptr};
  k_gemm<GSH, KTAIL, C, DR><<<dim3((unsigned)T, (unsigned)S), dim3(C::kThreads), C::kLdsBytes, s>>>(
      reinterpret_cast<const uint4*>(p->tiles), p->scales, p->sstride, p->tile_ptr, p->wpatch, X, Y, part, (int)M,
      (int)p->N, (int)p->K, Kt, (int)p->Nb, NT, T, per, dr);
  hipError_t e = hipGetLastError();
  if (S > 1) {
    if (e == hipSuccess) {
      e = launch_splitk_reduce(part, Y, M, p->N, S, s);
    }
    if (!ws) {
      const hipError_t f = hipFreeAsync(part, s);
      if (e == hipSuccess) e = f;
    }
  }
  return e;
}

}  // namespace

template <bool KTAIL, class C, bool DR>
hipError_t launch_g(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s, float* ws) {
  if (p->G == 128) return launch<0, KTAIL, C, DR>(p, X, M, Y, s, ws);
  if (p->G == 64) return launch<1, KTAIL, C, DR>(p, X, M, Y, s, ws);
  return launch<2, KTAIL, C, DR>(p, X, M, Y, s, ws);
}

// handles from mq_pack_blocks carry their residual as code tiles (DR)
template <bool KTAIL, class C>
hipError_t launch_d(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s, float* ws) {
  return p->blocks ? launch_g<KTAIL, C, true>(p, X, M, Y, s, ws) : launch_g<KTAIL, C, false>(p, X, M, Y, s, ws);
}

template <bool KTAIL>
hipError_t launch_k(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s, float* ws) {
  return M <= kNarrowMaxM ? launch_d<KTAIL, CfgNarrow>(p, X, M, Y, s, ws)
                          : launch_d<KTAIL, CfgWide>(p, X, M, Y, s, ws);
}

hipError_t launch_splitk_reduce(const float* part, uint16_t* Y, int64_t M, int64_t N, int S, hipStream_t s) {
  const int64_t quads = M * ((N + 3) / 4);
  k_splitk_reduce<<<dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s>>>(part, Y, (int)M, (int)N, S);
  return hipGetLastError();
}

hipError_t launch_gemm(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (M <= kGemmMidMaxM) return launch_gemm_mid(p, X, M, Y, s);
  if (gemm_rw_takes(p, M)) return launch_gemm_rw(p, X, M, Y, s);
  return (p->K % kTileCols) != 0 ? launch_k<true>(p, X, M, Y, s, nullptr) : launch_k<false>(p, X, M, Y, s, nullptr);
}

size_t gemm_workspace_bytes(const mq_packed* p, int64_t M) {
  if (M <= kGemmMidMaxM) return 0;   // the mid-size kernel splits K inside its workgroups
  if (gemm_rw_takes(p, M)) return 0;
  const int S = M <= kNarrowMaxM ? split_parts<CfgNarrow>(p, M, nullptr) : split_parts<CfgWide>(p, M, nullptr);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)p->N * sizeof(float) : 0;
}

hipError_t scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {   // first use on this device (it is current): its copy of the array
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_gemm_noalloc(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (M <= kGemmMidMaxM) return launch_gemm_mid(p, X, M, Y, s);   // no workspace
  if (gemm_rw_takes(p, M)) return launch_gemm_rw(p, X, M, Y, s);
  if (gemm_workspace_bytes(p, M) > kScratchBytes) return hipErrorInvalidValue;   // rejected by the caller first
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  float* w = static_cast<float*>(ws);
  return (p->K % kTileCols) != 0 ? launch_k<true>(p, X, M, Y, s, w) : launch_k<false>(p, X, M, Y, s, w);
}

size_t gemm_scratch_capacity() { return kScratchBytes; }

}  // namespace mq
