// Mid-size batch kernel (up to 64 tokens): Y = X (deq(Q_base) + deq(R))^T,
// fused, with no cross-workgroup workspace.
//
// ZipperEngine (MosaicQuant explainer, Methodology section 3) runs the sparse
// residual inside the dense 4-bit kernel. With a few dozen tokens the layer
// is a thin GEMM: too few output tiles to fill the chip unless K is split, and
// too few tokens per weight to amortise staging weights through LDS. Here:
//   * a workgroup of 8 waves owns R row blocks (16 R output features) and all
//     tokens of its slice; the waves split K (wave w takes code tiles w,
//     w + 8, ...), so the code tiles of a workgroup are read once, by one
//     wave each;
//   * a wave loads its code tiles straight into registers, a tile ahead of
//     their use, and widens them there to fp16(s q): the tile layout is the
//     A operand of the 16x16x32 fp16 MFMA as stored. X comes in with the
//     code tiles, with loads in which every 4 adjacent lanes read 64
//     contiguous bytes of one token row, and passes through a small per-wave
//     LDS slot into the B-operand layout (tokens as columns). Loading the B layout directly would have
//     each 4 adjacent lanes read 4 different token rows, which the L2-to-CU
//     path serves at well under half the rate, and every workgroup reads
//     all of X;
//   * the element-wise residual patches the widened registers through a
//     per-wave LDS plane laid out like the A operands: the lanes holding the
//     tile's entries write fp16(s q + sr qr) XOR fp16(s q) into it, every
//     lane XORs its own slice in (unpatched positions hold 0), and the
//     entries are cleared again; a block residual (Methodology section 2)
//     is a second code tile widened with its row scale and added in fp16;
//   * the 8 waves' partial sums meet in LDS and are added in wave order
//     (deterministic), then rounded once to fp16.
#include <algorithm>

#include "kernel_common.h"
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int kWavesM = 8;
constexpr int kThreadsM = 64 * kWavesM;
constexpr int kPlaneStrideM = 40;   // patch plane: halves per lane (80 B: 4 k-steps x 8, then 8 unused; 16 lanes
                                    // on distinct banks)
constexpr int kXSlotBytes = 4096;           // per wave: one token block's X for one code tile (16 x 128 fp16)
// Register sets in a wave's load ring: 2, or 3 for one row block and one
// token block per workgroup, where a wave's tiles (1 KiB each) are too small
// to keep enough bytes in flight (4096x11008 at 4 / 8 / 16 tokens: 15.3 /
// 15.4 / 15.7 us with 2, 13.8 / 13.9 / 15.1 with 3, 14.4 / 14.4 / 15.8 with
// 4); with more row blocks deeper rings measured slower at every shape.
template <int R, int NTB>
constexpr int mid_ring() { return R == 1 && NTB == 1 ? 3 : 2; }

// Residual of the handle: none; element-wise, either branch-free (kElemFlat1M
// + e - 1 when no tile's segment of the patch stream exceeds 64 e entries,
// e <= 3: each lane applies up to e entries per tile, all at once) or in
// rounds of 64 entries in a loop (kElemM, longer segments: the loop ties up
// enough registers that a workgroup takes at most 2 row blocks with 64
// tokens); or blocks of 4-bit codes.
enum { kPlainM = 0, kElemM = 1, kBlocksM = 2, kElemFlat1M = 3, kElemFlat3M = 5 };
constexpr bool is_flat(int mode) { return mode >= kElemFlat1M && mode <= kElemFlat3M; }
constexpr bool is_elem(int mode) { return mode == kElemM || is_flat(mode); }
constexpr int flat_entries(int mode) { return is_flat(mode) ? mode - kElemFlat1M + 1 : 1; }

// Reads of the patch plane, which is written 16 bits at a time, and its
// clearing: the type may alias anything, so the compiler keeps them in
// program order with the 16-bit writes (a wave's LDS operations then execute
// in that order).
typedef uint32_t plane_u32x4_t __attribute__((ext_vector_type(4), __may_alias__));

constexpr uint32_t kSelLoM = 0x05040100u, kSelHiM = 0x07060302u;
__device__ __forceinline__ half2_t splat_sel_m(uint32_t dword, uint32_t sel) {
  return __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(dword, dword, sel));
}

// Block residual as 4-bit code tiles (handles from mq_pack_blocks): slot of
// each (row block, tile), the tiles in the base layout, a scale per row.
struct DenseMid {
  const int32_t* slot;
  const uint4* tiles;
  const float* scale;
};

// Segment bounds (element-wise) or residual slot (kBlocksM) of the wave's code
// tiles, for the workgroup's row blocks: lane l holds those of the wave's
// tile l (wave + 8 l; a wave has at most 64 tiles as K <= 65536), loaded with
// one vector load per row block at the start. A step takes its tile's values
// out with readlane, so the loop issues no scalar loads: those share a
// completion counter with the LDS operations and return out of order, so
// every LDS wait would also wait for the scalar load just issued.
template <int R>
struct MidTab {
  uint32_t a[R], b[R];
};

template <int MODE, int R>
__device__ __forceinline__ void mid_table(MidTab<R>& tab, const uint32_t* __restrict__ tile_ptr,
                                          const DenseMid& dr, int Kt, int Nb, int rb0, int wave, int lane) {
  const int kl = min(wave + kWavesM * lane, Kt - 1);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int64_t t = (int64_t)min(rb0 + j, Nb - 1) * Kt + kl;
    if constexpr (MODE == kBlocksM) {
      tab.a[j] = (uint32_t)dr.slot[t];
      tab.b[j] = 0u;
    } else if constexpr (is_elem(MODE)) {
      tab.a[j] = tile_ptr[t];
      tab.b[j] = tile_ptr[t + 1];
    } else {
      tab.a[j] = tab.b[j] = 0u;
    }
  }
}

// The values of one tile (kt, the wave's tile idx): wave-uniform. Past the
// last tile the segment is empty and the slot that of the last tile.
template <int R>
struct MidPtrs {
  uint32_t p0[R], cnt[R];
};

template <int MODE, int R>
__device__ __forceinline__ void mid_ptrs(MidPtrs<R>& P, const MidTab<R>& tab, int Kt, int Nb, int rb0, int kt,
                                         int idx) {
  const int l = min(idx, 63);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if constexpr (MODE == kPlainM) {
      P.p0[j] = P.cnt[j] = 0u;
    } else {
      P.p0[j] = (uint32_t)__builtin_amdgcn_readlane((int)tab.a[j], l);
      if constexpr (is_elem(MODE)) {
        const uint32_t p1 = (uint32_t)__builtin_amdgcn_readlane((int)tab.b[j], l);
        P.cnt[j] = rb0 + j < Nb && kt < Kt ? p1 - P.p0[j] : 0u;
      } else {
        P.cnt[j] = 0u;
      }
    }
  }
}

// Everything one code tile needs, loaded a tile ahead of its use. Row blocks
// past the layer and tiles past K are clamped to the last ones (their
// results are never stored); rows past N have scale 0.
template <int GSH, int MODE, int NTB, int R>
struct MidTile {
  uint4 code[R];
  uint32_t sraw[R][GSH == 2 ? 2 : 1];   // the aligned scale word(s) of the lane's row holding the tile's scale(s)
  uint32_t ent[R][flat_entries(MODE)];  // element-wise: entries p0 + lane + 64 e; kBlocksM: [0] fp32 row scale
  uint32_t p0[R], cnt[R];               // element-wise: the tile's segment of the patch stream
  uint4 rcode[R];                       // kBlocksM
  u32x4_t x[NTB][4];                    // X as loaded: token block tb, load u (see mid_load)
};

template <int GSH, int MODE, int NTB, int R>
__device__ __forceinline__ void mid_load_base(MidTile<GSH, MODE, NTB, R>& T, const uint4* __restrict__ tiles,
                                              const uint16_t* __restrict__ scales, int64_t sstride,
                                              __amdgpu_buffer_rsrc_t xrs, const uint32_t (&xoff)[4], int K, int Kt,
                                              int Nb, int rb0, int kt, int lane) {
  const int r = lane & 15;
  const int ktc = min(kt, Kt - 1);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int rb = min(rb0 + j, Nb - 1);
    T.code[j] = tiles[((int64_t)rb * Kt + ktc) * 64 + lane];
    const uint16_t* srow = scales + (int64_t)(rb * kRowsPerBlock + r) * sstride;
    if constexpr (GSH == 0) {
      T.sraw[j][0] = reinterpret_cast<const uint32_t*>(srow)[ktc >> 1];
    } else if constexpr (GSH == 1) {
      T.sraw[j][0] = reinterpret_cast<const uint32_t*>(srow)[ktc];
    } else {
      const uint2 v = reinterpret_cast<const uint2*>(srow)[ktc];
      T.sraw[j][0] = v.x;
      T.sraw[j][1] = v.y;
    }
  }
  // The whole X offset (token row and column) goes into the per-lane offset,
  // which the buffer's range check covers: reads past the workgroup's last
  // row return zero, and so does all of X for a tile past the last (the
  // offset 2^30 is past any X range, and the sum cannot wrap), so such a tile
  // adds exactly zero.
  const uint32_t coff = kt < Kt ? (uint32_t)ktc * (kTileCols * 2) : (1u << 30);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[u] + coff + (uint32_t)tb * 32u * K, 0, 0);
      T.x[tb][u] = u32x4_t{v[0], v[1], v[2], v[3]};
    }
}

// The tile's residual: its patch entries (element-wise) or residual code tile and
// row scale (kBlocksM).
template <int GSH, int MODE, int NTB, int R>
__device__ __forceinline__ void mid_load_res(MidTile<GSH, MODE, NTB, R>& T, const MidPtrs<R>& P,
                                             const uint32_t* __restrict__ wpatch, const DenseMid& dr, int lane) {
  const int r = lane & 15;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if constexpr (is_elem(MODE)) {
#pragma unroll
      for (int e = 0; e < flat_entries(MODE); ++e)   // 1024 zero entries follow the stream: always readable
        T.ent[j][e] = wpatch[P.p0[j] + lane + 64 * e];
      T.p0[j] = P.p0[j];
      T.cnt[j] = P.cnt[j];
    } else if constexpr (MODE == kBlocksM) {
      T.rcode[j] = dr.tiles[(int64_t)P.p0[j] * 64 + lane];
      T.ent[j][0] = __builtin_bit_cast(uint32_t, dr.scale[(int64_t)P.p0[j] * kRowsPerBlock + r]);
    }
  }
}

// Element-wise residual of one row block's tile, applied to the widened A
// operands, one round of up to 64 entries (entries base .. base + 63 of the
// segment, entry base + lane in v). Entry bits (the patched-weight stream):
// 0-6 column mod 128, 11 valid, 12-15 row, 16-31 fp16(s q + sr qr) XOR
// fp16(s q). Its plane position is that of the weight in the A operands:
// lane r + 16 ((j % 32) / 8), k-step j / 32, element j % 8. Every lane writes
// (lanes without an entry to an unused part of their own slot), so the reads
// that follow see every lane's write.
__device__ __forceinline__ void mid_patch_round(half8_t (&a)[4], uint32_t v, uint32_t cnt, uint32_t base,
                                                uint16_t* plane, int lane) {
  const uint32_t c = v & 127u, row = (v >> 12) & 15u;
  uint32_t okm = 0u - (((uint32_t)lane + base < cnt) & ((v >> 11) & 1u));
  asm("" : "+v"(okm));
  const uint32_t real = (row + 16u * ((c >> 3) & 3u)) * kPlaneStrideM + 8u * (c >> 5) + (c & 7u);
  const uint32_t idle = (uint32_t)(lane * kPlaneStrideM + 32);
  const uint32_t tgt = idle ^ ((real ^ idle) & okm);
  plane[tgt] = (uint16_t)(v >> 16);
  const plane_u32x4_t* src = reinterpret_cast<const plane_u32x4_t*>(plane + lane * kPlaneStrideM);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4_t p = src[ks];
    a[ks] = __builtin_bit_cast(half8_t, __builtin_bit_cast(u32x4_t, a[ks]) ^ p);
  }
  plane[tgt] = 0;
}

// A segment of any length: rounds of 64 entries.
__device__ __forceinline__ void mid_patch(half8_t (&a)[4], uint32_t v, uint32_t cnt, uint32_t e0,
                                          const uint32_t* __restrict__ wpatch, uint16_t* plane, int lane) {
  for (uint32_t base = 0;;) {
    mid_patch_round(a, v, cnt, base, plane, lane);
    base += 64;
    if (base >= cnt) break;   // wave-uniform
    v = wpatch[e0 + base + lane];
  }
}

// A segment of up to 64 E entries, branch-free: lane l scatters entries
// l, l + 64, ... (each to its position, or to its own unused half past the
// end of the segment), then every lane reads its slice back once and the
// entries are cleared. Two entries never share a position (each names one
// weight).
template <int E>
__device__ __forceinline__ void mid_patch_flat(half8_t (&a)[4], const uint32_t (&v)[E], uint32_t cnt,
                                               uint16_t* plane, int lane) {
  const uint32_t idle = (uint32_t)(lane * kPlaneStrideM + 32);
  uint32_t tgt[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t c = v[e] & 127u, row = (v[e] >> 12) & 15u;
    uint32_t okm = 0u - (((uint32_t)(lane + 64 * e) < cnt) & ((v[e] >> 11) & 1u));
    asm("" : "+v"(okm));
    const uint32_t real = (row + 16u * ((c >> 3) & 3u)) * kPlaneStrideM + 8u * (c >> 5) + (c & 7u);
    tgt[e] = idle ^ ((real ^ idle) & okm);
    plane[tgt[e]] = (uint16_t)(v[e] >> 16);
  }
  const plane_u32x4_t* src = reinterpret_cast<const plane_u32x4_t*>(plane + lane * kPlaneStrideM);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4_t p = src[ks];
    a[ks] = __builtin_bit_cast(half8_t, __builtin_bit_cast(u32x4_t, a[ks]) ^ p);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) plane[tgt[e]] = 0;
}

template <int GSH, int MODE, int NTB, int R, bool KTAIL>
__device__ __forceinline__ void mid_compute(float4_t (&acc)[R][NTB], const MidTile<GSH, MODE, NTB, R>& T,
                                            const uint32_t* __restrict__ wpatch, int kt,
                                            uint16_t* plane, plane_u32x4_t* xslot, const uint32_t (&xpos)[4],
                                            int K, int Kt, int lane, uint32_t vmask, uint32_t vmask4,
                                            uint32_t vmagic) {
  // X into the B-operand layout through the wave's slot, one token block at
  // a time (a wave's LDS operations execute in program order, so each block's
  // reads see its writes and finish before the next block's writes)
  half8_t xb[NTB][4];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) xslot[64 * u + lane] = T.x[tb][u];
#pragma unroll
    for (int t = 0; t < 4; ++t) xb[tb][t] = __builtin_bit_cast(half8_t, xslot[xpos[t]]);
  }
  if constexpr (KTAIL) {
    // columns past K (a K tail) are zeroed: they meet weights 0, but another
    // row's values there need not be finite (every tile, branch-free: a
    // branch here costs registers)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t keep = kt * kTileCols + 32 * t + 8 * (lane >> 4) < K ? ~0u : 0u;
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const u32x4_t v = __builtin_bit_cast(u32x4_t, xb[tb][t]);
        xb[tb][t] = __builtin_bit_cast(half8_t, u32x4_t{v[0] & keep, v[1] & keep, v[2] & keep, v[3] & keep});
      }
    }
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    half2_t s[4];
    if constexpr (GSH == 0) {
      s[0] = s[1] = s[2] = s[3] = splat_sel_m(T.sraw[j][0], (kt & 1) ? kSelHiM : kSelLoM);
    } else if constexpr (GSH == 1) {
      s[0] = s[1] = splat_sel_m(T.sraw[j][0], kSelLoM);
      s[2] = s[3] = splat_sel_m(T.sraw[j][0], kSelHiM);
    } else {
      s[0] = splat_sel_m(T.sraw[j][0], kSelLoM);
      s[1] = splat_sel_m(T.sraw[j][0], kSelHiM);
      s[2] = splat_sel_m(T.sraw[j][1], kSelLoM);
      s[3] = splat_sel_m(T.sraw[j][1], kSelHiM);
    }
    half8_t a[4];
    a[0] = dequant_dword(T.code[j].x, s[0], vmask, vmask4, vmagic);
    a[1] = dequant_dword(T.code[j].y, s[1], vmask, vmask4, vmagic);
    a[2] = dequant_dword(T.code[j].z, s[2], vmask, vmask4, vmagic);
    a[3] = dequant_dword(T.code[j].w, s[3], vmask, vmask4, vmagic);
    if constexpr (MODE == kBlocksM) {
      const _Float16 sr = (_Float16)__builtin_bit_cast(float, T.ent[j][0]);
      const half2_t srs = {sr, sr};
      a[0] += dequant_dword(T.rcode[j].x, srs, vmask, vmask4, vmagic);
      a[1] += dequant_dword(T.rcode[j].y, srs, vmask, vmask4, vmagic);
      a[2] += dequant_dword(T.rcode[j].z, srs, vmask, vmask4, vmagic);
      a[3] += dequant_dword(T.rcode[j].w, srs, vmask, vmask4, vmagic);
    } else if constexpr (is_flat(MODE)) {
      mid_patch_flat<flat_entries(MODE)>(a, T.ent[j], T.cnt[j], plane, lane);
    } else if constexpr (MODE == kElemM) {
      if (T.cnt[j] != 0u) mid_patch(a, T.ent[j][0], T.cnt[j], T.p0[j], wpatch, plane, lane);
    }
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc[j][tb] = mfma16(a[ks], xb[tb][ks], acc[j][tb]);
  }
  // The accumulators may be copied right after this point, in another basic
  // block (the loop's exit after an odd number of tiles), where the compiler
  // was seen to read the last MFMAs' results without the wait states an MFMA
  // result needs before a VALU reads it: 16 of them here, unconditionally.
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7");
}

template <int GSH, int MODE, int NTB, int R, bool KTAIL>
__global__ __launch_bounds__(kThreadsM, 1) void k_gemm_mid(const uint4* __restrict__ tiles,
                                                           const uint16_t* __restrict__ scales, int64_t sstride,
                                                           const uint32_t* __restrict__ tile_ptr,
                                                           const uint32_t* __restrict__ wpatch, DenseMid dr,
                                                           const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                           int M, int N, int K, int Kt, int Nb) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_mid[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rb0 = blockIdx.x * R, m0 = blockIdx.y * 16 * NTB;
  uint16_t* const plane = reinterpret_cast<uint16_t*>(lds_mid) + wave * 64 * kPlaneStrideM;
  constexpr int xbase = is_elem(MODE) ? kWavesM * 64 * kPlaneStrideM * 2 : 0;   // the X slots follow the planes
  plane_u32x4_t* const xslot = reinterpret_cast<plane_u32x4_t*>(lds_mid + xbase + wave * kXSlotBytes);
  if constexpr (is_elem(MODE)) {
    // LDS holds whatever a previous kernel left: each lane zeroes the 32
    // halves of its slot that the patches XOR in
    plane_u32x4_t* dst = reinterpret_cast<plane_u32x4_t*>(plane + lane * kPlaneStrideM);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) dst[ks] = plane_u32x4_t{0u, 0u, 0u, 0u};
  }
  // X through a buffer resource over the workgroup's token rows: rows past M
  // read as zero
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + (int64_t)m0 * K), 0, (int)(min(16 * NTB, M - m0) * K * 2), kBufferRaw);
  uint32_t xoff[4], xpos[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    xoff[u] = ((uint32_t)(4 * u + (lane >> 4)) * (uint32_t)K + 8u * x_load_chunk(lane, u)) * 2u;
    xpos[u] = x_read_pos(lane, u);
  }
  uint32_t vmask = 0x000F000Fu, vmask4 = 0x00F000F0u, vmagic = 0x64006400u;
  asm volatile("" : "+v"(vmask), "+v"(vmask4), "+v"(vmagic));   // keep the constants in VGPRs for v_and_or_b32

  // The accumulators start from a zero the compiler cannot see through: with
  // a literal zero it was seen to rematerialise only some components of an
  // accumulator (the others holding whatever the registers last held).
  float z = 0.f;
  asm volatile("" : "+v"(z));
  float4_t acc[R][NTB];
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[j][tb] = float4_t{z, z, z, z};

  // Tiles wave, wave + 8, ...: a ring of kRingM register sets, each loaded
  // kRingM - 1 tiles ahead of its use, in whole turns of the ring with no branch inside
  // (one costs registers): the steps past the wave's last tile compute on
  // zero X. The segment table is requested first; the first tiles' residual
  // loads, which need it, follow their code tiles.
  constexpr int kRingM = mid_ring<R, NTB>();
  MidTab<R> tab;
  mid_table<MODE, R>(tab, tile_ptr, dr, Kt, Nb, rb0, wave, lane);
  MidTile<GSH, MODE, NTB, R> T[kRingM];
#pragma unroll
  for (int u = 0; u + 1 < kRingM; ++u)
    mid_load_base<GSH, MODE, NTB, R>(T[u], tiles, scales, sstride, xrs, xoff, K, Kt, Nb, rb0, wave + kWavesM * u,
                                     lane);
#pragma unroll
  for (int u = 0; u + 1 < kRingM; ++u) {
    MidPtrs<R> P;
    mid_ptrs<MODE, R>(P, tab, Kt, Nb, rb0, wave + kWavesM * u, u);
    mid_load_res<GSH, MODE, NTB, R>(T[u], P, wpatch, dr, lane);
  }
  const int nt = (Kt - wave + kWavesM - 1) / kWavesM;   // tiles of this wave
  for (int i = 0; i < nt; i += kRingM) {
#pragma unroll
    for (int u = 0; u < kRingM; ++u) {
      const int kt = wave + kWavesM * (i + u), kn = kt + kWavesM * (kRingM - 1);
      MidPtrs<R> P;
      mid_ptrs<MODE, R>(P, tab, Kt, Nb, rb0, kn, i + u + kRingM - 1);
      MidTile<GSH, MODE, NTB, R>& Tn = T[(u + kRingM - 1) % kRingM];
      mid_load_base<GSH, MODE, NTB, R>(Tn, tiles, scales, sstride, xrs, xoff, K, Kt, Nb, rb0, kn, lane);
      mid_load_res<GSH, MODE, NTB, R>(Tn, P, wpatch, dr, lane);
      mid_compute<GSH, MODE, NTB, R, KTAIL>(acc, T[u], wpatch, kt, plane, xslot, xpos, K, Kt, lane, vmask, vmask4,
                                            vmagic);
    }
  }

  // The 8 partial sums of each (row block, token block) meet in LDS (the
  // planes' and slots' space, once every wave is done with it) and are added
  // in wave order. Lane l = n + 16 g holds D[4 g + i][n]: output features
  // 4 g + i of the row block, token n of the token block.
  float4_t* red = reinterpret_cast<float4_t*>(lds_mid);   // [R * NTB][8 waves][64]
  __syncthreads();
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) red[((j * NTB + tb) * kWavesM + wave) * 64 + lane] = acc[j][tb];
  __syncthreads();
  for (int c = wave; c < R * NTB; c += kWavesM) {
    const int j = c / NTB, tb = c - j * NTB;
    float4_t sum = red[(c * kWavesM) * 64 + lane];
#pragma unroll
    for (int w = 1; w < kWavesM; ++w) sum += red[(c * kWavesM + w) * 64 + lane];
    const int m = m0 + 16 * tb + (lane & 15);
    const int n0 = (rb0 + j) * kRowsPerBlock + 4 * (lane >> 4);
    if (m < M && rb0 + j < Nb && n0 < N) store4(Y + (int64_t)m * N + n0, sum, N - n0, (N & 3) == 0);
  }
}

template <int GSH, int MODE, int NTB, int R, bool KTAIL>
hipError_t launch_mid(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  constexpr size_t work_bytes = (is_elem(MODE) ? (size_t)kWavesM * 64 * kPlaneStrideM * 2 : 0) +
                                (size_t)kWavesM * kXSlotBytes;
  constexpr size_t red_bytes = (size_t)R * NTB * kWavesM * 64 * sizeof(float4_t);
  constexpr size_t lds = work_bytes > red_bytes ? work_bytes : red_bytes;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_mid<GSH, MODE, NTB, R, KTAIL>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const DenseMid dr = MODE == kBlocksM ? DenseMid{p->rt_slot, reinterpret_cast<const uint4*>(p->rt_tiles), p->bscale}
                                       : DenseMid{nullptr, nullptr, nullptr};
  const dim3 grid((unsigned)((p->Nb + R - 1) / R), (unsigned)((M + 16 * NTB - 1) / (16 * NTB)));
  k_gemm_mid<GSH, MODE, NTB, R, KTAIL><<<grid, dim3(kThreadsM), lds, s>>>(
      reinterpret_cast<const uint4*>(p->tiles), p->scales, p->sstride, p->tile_ptr, p->wpatch, dr, X, Y, (int)M,
      (int)p->N, (int)p->K, (int)p->Kt, (int)p->Nb);
  return hipGetLastError();
}

// Row blocks per workgroup: enough that one round of workgroups covers the
// layer on 256 CUs (fewer row blocks per workgroup would make a second
// round, each reading all of its X again), at most 4; with 64 tokens 2 for
// the looping element-wise residual or a K tail, and 3 with G = 32 for a
// block residual or 3 patch entries per lane, where more would not fit the
// registers.
template <int GSH, int MODE, int NTB, bool KTAIL>
hipError_t launch_mid_r(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  constexpr int64_t rmax = NTB < 4                                                  ? 4
                           : (MODE == kElemM || KTAIL)                               ? 2
                           : (MODE == kBlocksM || MODE == kElemFlat3M) && GSH == 2 ? 3
                                                                                     : 4;
  const int64_t r = std::min<int64_t>(rmax, std::max<int64_t>(1, (p->Nb + 255) / 256));
  if (r == 1) return launch_mid<GSH, MODE, NTB, 1, KTAIL>(p, X, M, Y, s);
  if (r == 2 || rmax == 2) return launch_mid<GSH, MODE, NTB, 2, KTAIL>(p, X, M, Y, s);
  if constexpr (rmax >= 3) {
    if (r == 3 || rmax == 3) return launch_mid<GSH, MODE, NTB, 3, KTAIL>(p, X, M, Y, s);
  }
  if constexpr (rmax >= 4) return launch_mid<GSH, MODE, NTB, 4, KTAIL>(p, X, M, Y, s);
  return hipErrorInvalidValue;   // not reached
}

template <int GSH, int MODE, bool KTAIL>
hipError_t launch_mid_n(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (M <= 16) return launch_mid_r<GSH, MODE, 1, KTAIL>(p, X, M, Y, s);
  if (M <= 32) return launch_mid_r<GSH, MODE, 2, KTAIL>(p, X, M, Y, s);
  return launch_mid_r<GSH, MODE, 4, KTAIL>(p, X, M, Y, s);
}

template <int MODE, bool KTAIL>
hipError_t launch_mid_g(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (p->G == 128) return launch_mid_n<0, MODE, KTAIL>(p, X, M, Y, s);
  if (p->G == 64) return launch_mid_n<1, MODE, KTAIL>(p, X, M, Y, s);
  return launch_mid_n<2, MODE, KTAIL>(p, X, M, Y, s);
}

template <bool KTAIL>
hipError_t launch_mid_m(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (p->blocks) {
    return p->nblk > 0 ? launch_mid_g<kBlocksM, KTAIL>(p, X, M, Y, s) : launch_mid_g<kPlainM, KTAIL>(p, X, M, Y, s);
  }
  if (p->nnz == 0) return launch_mid_g<kPlainM, KTAIL>(p, X, M, Y, s);
  if (p->max_seg <= 64) return launch_mid_g<kElemFlat1M, KTAIL>(p, X, M, Y, s);
  if (p->max_seg <= 128) return launch_mid_g<kElemFlat1M + 1, KTAIL>(p, X, M, Y, s);
  if (p->max_seg <= 192) return launch_mid_g<kElemFlat3M, KTAIL>(p, X, M, Y, s);
  return launch_mid_g<kElemM, KTAIL>(p, X, M, Y, s);
}

}  // namespace

hipError_t launch_gemm_mid(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  return (p->K % kTileCols) != 0 ? launch_mid_m<true>(p, X, M, Y, s) : launch_mid_m<false>(p, X, M, Y, s);
}

}  // namespace mq
