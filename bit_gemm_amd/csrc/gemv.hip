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

namespace mq {
namespace {

constexpr int kWaves = 8;
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
                                            const int64_t (&srow)[4], const bool (&rowok)[4], int kt) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t si = srow[i] + (int64_t)kt * NS;
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
                                         int K, int kt, int g, uint32_t vmask, uint32_t vmagic) {
  constexpr int SPG = 4 / NS;   // MFMA k-steps per scale group
  half8_t a[4];
  a[0] = widen_q(code.x, vmask, vmagic);
  a[1] = widen_q(code.y, vmask, vmagic);
  a[2] = widen_q(code.z, vmask, vmagic);
  a[3] = widen_q(code.w, vmask, vmagic);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    half8_t bx[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int seg = kt * kTileCols + 32 * s4;
      if (PAD && seg >= K)   // padded 32-column segment (uniform branch)
        bx[s4] = as_half8(make_uint4(0u, 0u, 0u, 0u));
      else if (XLDS)
        bx[s4] = *reinterpret_cast<const half8_t*>(xs + mrow[mb] * K + seg + 8 * g);
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

// GSH = log2(128 / G). XLDS: X staged whole in LDS (M * K * 2 bytes), else X
// fragments come from global memory. MW: K > 4096 (several column windows).
// TPW > 0: every wave owns exactly TPW tiles (Kt == 8 TPW, K % 128 == 0) and
// loads them all up front; TPW == 0: any shape, one tile per iteration.
template <int MB, int GSH, bool XLDS, bool MW, int TPW>
__global__ __launch_bounds__(64 * kWaves) void k_gemv(const uint4* __restrict__ tiles,
                                                      const uint16_t* __restrict__ scales, int64_t sstride,
                                                      const uint32_t* __restrict__ tile_ptr,
                                                      const uint32_t* __restrict__ entries,
                                                      const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                      int M, int N, int K, int Kt) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [M][K] when XLDS
  __shared__ float4_t red[kWaves][MB][64];
  constexpr int NS = 1 << GSH;
  const int rb = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int kt0 = TPW ? wave * TPW : (Kt * wave) / kWaves;
  const int kt1 = TPW ? kt0 + TPW : (Kt * (wave + 1)) / kWaves;
  const int64_t tbase = (int64_t)rb * Kt;
  int mrow[MB];
  token_rows<MB>(M, r, mrow);

  // ---- residual entries of this wave's first two chunks (issued first)
  const uint32_t E0 = tile_ptr[tbase], E1 = tile_ptr[tbase + Kt];
  uint32_t ent[2][8];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t idx = E0 + 32u * (uint32_t)(wave + kWaves * c) + 8u * g + u;
      ent[c][u] = (idx < E1) ? entries[idx] : 0u;   // entry 0: zero value
    }

  int64_t srow[4];
  bool rowok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rb * kRowsPerBlock + 4 * g + i;
    rowok[i] = row < N;
    srow[i] = (int64_t)min(row, N - 1) * sstride;
  }

  // ---- all code tiles of the wave (fast path) issued before anything waits
  constexpr int NT = TPW ? TPW : 1;
  uint4 code[NT];
  TileScales<NS> S[NT];
  if (TPW) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      code[t] = tiles[(tbase + kt0 + t) * 64 + lane];
      load_scales<NS>(S[t], scales, srow, rowok, kt0 + t);
    }
  }
  if (XLDS) {
    const int n16 = (M * K) >> 3;
    const uint4* src = reinterpret_cast<const uint4*>(X);
    uint4* dst = reinterpret_cast<uint4*>(xs);
    for (int i = threadIdx.x; i < n16; i += 64 * kWaves) dst[i] = src[i];
    __syncthreads();
  }

  uint32_t vmask = 0x000F000Fu, vmagic = 0x64006400u;
  asm volatile("" : "+v"(vmask), "+v"(vmagic));   // keep both constants in VGPRs for v_and_or_b32

  float4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
  if (TPW) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      tile_mma<MB, NS, XLDS, false>(acc, code[t], S[t], X, xs, mrow, K, kt0 + t, g, vmask, vmagic);
  } else {
    for (int kt = kt0; kt < kt1; ++kt) {
      const uint4 c1 = tiles[(tbase + kt) * 64 + lane];
      TileScales<NS> s1;
      load_scales<NS>(s1, scales, srow, rowok, kt);
      tile_mma<MB, NS, XLDS, true>(acc, c1, s1, X, xs, mrow, K, kt, g, vmask, vmagic);
    }
  }

  // ---- residual: chunks wave, wave + 8, ... of the row block's entries
  const uint32_t nchunks = (E1 - E0 + 31u) >> 5;
  const int nwin = (Kt + 31) >> 5;
  for (uint32_t c = (uint32_t)wave, ci = 0; c < nchunks; c += kWaves, ++ci) {
    uint32_t e[8];
    if (ci < 2) {
#pragma unroll
      for (int u = 0; u < 8; ++u) e[u] = (ci == 0) ? ent[0][u] : ent[1][u];
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t idx = E0 + 32u * c + 8u * g + u;
        e[u] = (idx < E1) ? entries[idx] : 0u;
      }
    }
    int col[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      int wb = 0;
      if (MW) {
        const uint32_t idx = E0 + 32u * c + 8u * g + u;
        for (int w = 1; w < nwin; ++w) wb += (idx >= tile_ptr[tbase + 32 * w]) ? kColWindow : 0;
      }
      col[u] = wb + (int)ent_col(e[u]);
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
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        uint32_t lo, hi;
        if (XLDS) {
          lo = xs[mrow[mb] * K + col[u]];
          hi = xs[mrow[mb] * K + col[u + 1]];
        } else {
          lo = X[(int64_t)mrow[mb] * K + col[u]];
          hi = X[(int64_t)mrow[mb] * K + col[u + 1]];
        }
        bv[u >> 1] = lo | (hi << 16);
      }
      acc[mb] = mfma16(a, __builtin_bit_cast(half8_t, bv), acc[mb]);
    }
  }

  // ---- fixed-order sum of the 8 partial tiles, fp16 output
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  if (wave < MB) {
    const int mb = wave;
    float4_t s = red[0][mb][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += red[w][mb][lane];
    const int m = mb * 16 + r;                   // token
    const int n0 = rb * kRowsPerBlock + 4 * g;   // first of 4 output features
    if (m < M) store4(Y + (int64_t)m * N + n0, s, N - n0, (N & 3) == 0);
  }
}

constexpr size_t kXldsMax = 64 * 1024;

template <int MB, int GSH, bool XL, bool MWV, int TPW>
hipError_t launch(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s, size_t xbytes) {
  if (XL) {
    static bool done = false;   // once per instantiation: allow 64 KiB of dynamic LDS
    if (!done) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<MB, GSH, XL, MWV, TPW>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kXldsMax);
      if (e != hipSuccess) return e;
      done = true;
    }
  }
  k_gemv<MB, GSH, XL, MWV, TPW><<<dim3((unsigned)p->Nb), dim3(64 * kWaves), XL ? xbytes : 0, s>>>(
      reinterpret_cast<const uint4*>(p->tiles), p->scales, p->sstride, p->tile_ptr, p->entries, X, Y, M,
      (int)p->N, (int)p->K, (int)p->Kt);
  return hipGetLastError();
}

template <int MB, int GSH, bool XL, bool MWV>
hipError_t pick_tpw(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s, size_t xbytes) {
  const bool exact = (p->K % kTileCols) == 0 && (p->Kt % kWaves) == 0;
  const int64_t tpw = p->Kt / kWaves;
  if (exact && tpw == 4) return launch<MB, GSH, XL, MWV, 4>(p, X, M, Y, s, xbytes);
  if (exact && tpw == 8) return launch<MB, GSH, XL, MWV, 8>(p, X, M, Y, s, xbytes);
  if (exact && tpw == 2) return launch<MB, GSH, XL, MWV, 2>(p, X, M, Y, s, xbytes);
  if (exact && tpw == 1) return launch<MB, GSH, XL, MWV, 1>(p, X, M, Y, s, xbytes);
  return launch<MB, GSH, XL, MWV, 0>(p, X, M, Y, s, xbytes);
}

template <int MB, int GSH>
hipError_t run(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  const size_t xbytes = (size_t)M * p->K * 2;
  const bool xlds = MB == 1 && xbytes <= kXldsMax;
  const bool mw = p->Kt > 32;
  if (xlds) return mw ? pick_tpw<MB, GSH, true, true>(p, X, M, Y, s, xbytes)
                      : pick_tpw<MB, GSH, true, false>(p, X, M, Y, s, xbytes);
  return mw ? pick_tpw<MB, GSH, false, true>(p, X, M, Y, s, xbytes)
            : pick_tpw<MB, GSH, false, false>(p, X, M, Y, s, xbytes);
}

template <int MB>
hipError_t run_g(const mq_packed* p, const uint16_t* X, int M, uint16_t* Y, hipStream_t s) {
  if (p->G == 128) return run<MB, 0>(p, X, M, Y, s);
  if (p->G == 64) return run<MB, 1>(p, X, M, Y, s);
  return run<MB, 2>(p, X, M, Y, s);
}

}  // namespace

hipError_t launch_gemv(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (M <= 16) return run_g<1>(p, X, (int)M, Y, s);
  if (M <= 32) return run_g<2>(p, X, (int)M, Y, s);
  return run_g<4>(p, X, (int)M, Y, s);
}

}  // namespace mq
