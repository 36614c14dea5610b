// 4-bit activations (W4A4): the activation quantizer and the fused W4A4 linear.
//
// MosaicQuant explainer, Experimental Results (Accuracy): the method is
// evaluated with 4-bit weights and 4-bit activations. Methodology section 3
// (ZipperEngine): quantization is one stage of the overlapped pipeline, next
// to the dense compute, the sparse compensation and the reduction-add.
//
// Activations are quantized like the base weights, per token and per group of
// G input columns: sx = fp16(max |x| / 7), qx = clamp(rne(x / sx), -7, 7),
// decided exactly with 32-bit arithmetic (fp16_div7_h, quant7_f in
// quant_exact.h).
//
// Matrix cores. gfx950's 16x16x128 fp8 MFMA multiplies 32 bytes per lane of
// each operand and accumulates in fp32; on 4-bit integers its products and
// sums are exact. Neither operand needs arithmetic to get there:
//   * weights: the nibbles of a code tile split into bytes. A byte holding
//     u in [0, 15] is, read as OCP e4m3, exactly u 2^-9 (subnormal below 8),
//     so d & 0x0F0F0F0F and (d >> 4) & 0x0F0F0F0F are fp8 operands;
//   * activations: qx stored by the quantizer as e4m3 bytes, in the order in
//     which the split nibbles arrive ("tile order", below).
// One MFMA gives 2^-9 sum_k u_k qx_k over one 128-column tile. The weight
// offset u = q + 8 is removed through the accumulator input C = -2^-6 sum qx
// (per token and group), so D = 2^-9 sum q qx exactly; the group's part is
// then added in fp32 as acc += D * (512 sx * s): two VALU ops per output.
// Groups narrower than a tile take one MFMA each, with the activation bytes
// of the other groups zeroed.
//
// Tile order: for token m and column tile kt, byte 32 g + 8 t + p of the
// tile's 128 bytes holds the code of column 128 kt + 32 t + 8 g + perm[p],
// perm = {0, 4, 1, 5, 2, 6, 3, 7} (lane group g of the weight tile holds the
// same columns, nibble by nibble, in the same order after the split).
//
// Block residual (handles from mq_pack_blocks, Methodology section 2): a
// selected block is a second 16 x 128 code tile with a scale sr per row; it
// takes the same activation operand and C and adds D * (512 sx * sr). Blocks
// are 16 rows, one wave's row block, so the test is uniform in the wave.
#include <algorithm>
#include <type_traits>

#include "kernel_common.h"
#include "mq_internal.h"
#include "quant_exact.h"

namespace mq {
namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kBn = 256;                 // output features per workgroup (16 row blocks)
constexpr int kLdsRow = 144;             // bytes per staged token row: 128 + 16, so 8 rows hit distinct banks
constexpr int kSplitTarget = 256;        // workgroups to aim for when K is split
constexpr int kE8m0One = 127;            // MFMA block scale 2^0
constexpr uint32_t kNibbleBytes = 0x0F0F0F0Fu;

// ------------------------------------------------------------- quantizer

// e4m3 byte of a code q in [-7, 7] (exact: 1 = 0x38, 2..3 = 0x40 | .., 4..7 = 0x48 | ..)
__device__ __forceinline__ uint32_t e4m3_code(int q) {
  const uint32_t a = (uint32_t)(q < 0 ? -q : q);
  const uint32_t v = a == 0u ? 0u : a == 1u ? 0x38u : a < 4u ? (0x40u | ((a - 2u) << 2)) : (0x48u | ((a - 4u) << 1));
  return v | (q < 0 ? 0x80u : 0u);
}

// One lane per 8 columns of a token row (chunk c = 4 g + t of a tile: the
// tile-order bytes 8 c .. 8 c + 7). The 16 chunks of a (token, tile) are 16
// consecutive lanes, all active; a group's chunks differ in g (all G), in t's
// low bit (G >= 64) and in t's high bit (G = 128), and reduce over those
// lanes. Writes the chunk's 8 codes at xq_tile + 8 c (the tile's 128 bytes
// of token m) and the group metadata at meta_tile[0 .. NG) (token m, tile kt).
// v: the chunk's 8 fp16 values (zero past K).
template <int NG>
__device__ __forceinline__ void quant_chunk_v(uint4 v, int c, uint8_t* xq_tile, uint32_t* meta_tile) {
  const int g = c >> 2, t = c & 3;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
  uint32_t amax = 0u;   // magnitude bits: ordered like the values; >= 0x7C00 for inf / NaN
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = max(amax, h[i] & 0x7FFFu);
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 4));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 8));
  if (NG <= 2) amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  if (NG == 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  // a group with a non-finite entry gets a NaN scale (its outputs become NaN) and zero codes
  const bool finite = amax < 0x7C00u;
  const uint32_t sbits = finite ? fp16_div7_h(amax) : 0x7E00u;
  const float sf = finite ? h_to_f(sbits) : 0.0f;
  int q[8];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    q[i] = quant7_f(h_to_f(h[i]), sf);
    sum += q[i];
  }
  const uint32_t lo = e4m3_code(q[0]) | (e4m3_code(q[4]) << 8) | (e4m3_code(q[1]) << 16) | (e4m3_code(q[5]) << 24);
  const uint32_t hi = e4m3_code(q[2]) | (e4m3_code(q[6]) << 8) | (e4m3_code(q[3]) << 16) | (e4m3_code(q[7]) << 24);
  *reinterpret_cast<uint2*>(xq_tile + 8 * c) = make_uint2(lo, hi);
  sum += __shfl_xor(sum, 4);
  sum += __shfl_xor(sum, 8);
  if (NG <= 2) sum += __shfl_xor(sum, 1);
  if (NG == 1) sum += __shfl_xor(sum, 2);
  constexpr int TPG = 4 / NG;   // t values per group
  if (g == 0 && (t % TPG) == 0) meta_tile[t / TPG] = sbits | ((uint32_t)(sum & 0xFFFF) << 16);
}

template <int NG>
__device__ __forceinline__ void quant_chunk(const uint16_t* __restrict__ X, int K, int m, int kt, int c,
                                            uint8_t* xq_tile, uint32_t* meta_tile) {
  const int col0 = 128 * kt + 32 * (c & 3) + 8 * (c >> 2);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (col0 < K) v = *reinterpret_cast<const uint4*>(X + (int64_t)m * K + col0);
  quant_chunk_v<NG>(v, c, xq_tile, meta_tile);
}

// The quantizer kernel: one thread per chunk of every (token, tile).
template <int NG>
__global__ __launch_bounds__(256) void k_quant_a4(const uint16_t* __restrict__ X, int M, int K, int Kt,
                                                  uint8_t* __restrict__ xq, uint32_t* __restrict__ xmeta) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t unit = gid >> 4;                      // (token, tile); the 16 lanes exit together
  if (unit >= (int64_t)M * Kt) return;
  const int c = (int)(gid & 15);
  const int m = (int)(unit / Kt), kt = (int)(unit - (int64_t)m * Kt);
  const int64_t Kp = (int64_t)Kt * kTileCols;
  quant_chunk<NG>(X, K, m, kt, c, xq + (int64_t)m * Kp + 128 * kt, xmeta + ((int64_t)m * Kt + kt) * NG);
}

// ------------------------------------------------------------- W4A4 GEMM

// Workgroup: 256 features x BM tokens, NWN x NWM waves; a wave owns RB = 16 /
// NWN row blocks (16 features each) and MS 16-token slices.
template <int NWN_, int NWM_, int MS_>
struct CfgA4 {
  static constexpr int kNwn = NWN_, kNwm = NWM_, kMs = MS_;
  static constexpr int kWaves = NWN_ * NWM_;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRb = 16 / NWN_;
  static constexpr int kBm = 16 * MS_ * NWM_;
  static constexpr int kChunks = kBm * 8;                          // 16-byte chunks of a staged activation tile
  static constexpr int kXr = (kChunks + kThreads - 1) / kThreads;   // chunks per thread
  static constexpr int kMinBlocks = 2;                              // workgroups per CU
  static_assert(16 % NWN_ == 0 && MS_ >= 1, "workgroup shape");
};
// 256 x 64 with waves of 32 x 64 (up to 128 VGPRs, so two workgroups share a
// CU: a larger tile of 8 waves leaves one wave's MFMA-to-VALU dependencies
// exposed, and the second workgroup's waves fill them). Up to 16 tokens run
// the decode kernel below instead.
using CfgA4Mid = CfgA4<8, 1, 4>;

template <int NG, int BM>
struct StageA4 {
  // [BM][kLdsRow] codes, then [NG][BM] fp32 512 sx, then [NG][BM] fp32 C = -2^-6 sum qx
  static constexpr int kScaleOff = BM * kLdsRow;
  static constexpr int kCOff = kScaleOff + NG * BM * 4;
  static constexpr int kBytes = kCOff + NG * BM * 4;
};

// Block residual kept as code tiles: slot[rb * Kt + kt] (nblk where none),
// tiles in the base tile layout, one fp32 scale per row.
struct DenseA4 {
  const int32_t* slot;
  const uint4* tiles;
  const float* scale;
  int nblk;
};

// The handle's arrays (pointer, bytes) for the buffer resources the kernel
// builds: every weight-side load is then a wave-uniform byte offset (SGPR)
// plus one per-lane offset fixed for the whole kernel, so no per-load 64-bit
// addresses occupy VGPRs.
struct WArrays {
  const void* tiles;
  const void* scales;
  const void* rtiles;
  const void* rscale;
  int tiles_b, scales_b, rtiles_b, rscale_b;
  uint32_t sstride_b;   // bytes per scale row
};
struct WSrc {
  __amdgpu_buffer_rsrc_t tiles, scales, rtiles, rscale;
  uint32_t sstride_b;
};
__device__ __forceinline__ WSrc make_wsrc(const WArrays& a) {
  WSrc s;
  s.tiles = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.tiles), 0, a.tiles_b, kBufferRaw);
  s.scales = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.scales), 0, a.scales_b, kBufferRaw);
  s.rtiles = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.rtiles), 0, a.rtiles_b, kBufferRaw);
  s.rscale = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.rscale), 0, a.rscale_b, kBufferRaw);
  s.sstride_b = a.sstride_b;
  return s;
}

template <int RB, int NG>
struct WRegs {
  using SrawT = std::conditional_t<NG == 4, uint2, uint32_t>;
  uint4 code[RB];   // the lane's 16 bytes of the base code tile
  SrawT sraw[RB];   // aligned scale dword(s) of the lane's row holding this tile's group scales
  uint4 rcode[RB];  // block residual: the same 16 bytes of the residual tile (its slot's)
  float rsc[RB];    // residual scale of the lane's row
  int slot[RB];     // residual slot (wave-uniform)
};

template <int RB>
__device__ __forceinline__ void load_slots(int (&sl)[RB], const DenseA4& dr, int Kt, int Nb, int rbw, int kt) {
#pragma unroll
  for (int j = 0; j < RB; ++j)
    sl[j] = __builtin_amdgcn_readfirstlane(dr.slot[(int64_t)min(rbw + j, Nb - 1) * Kt + min(kt, Kt - 1)]);
}

// Loads only (no selects on loaded values): row blocks past the layer and
// tiles past K are clamped and feed nothing that is stored. vcode = 16 lane,
// vscale = (lane % 16) * row stride, vrs = 4 (lane % 16).
template <int NG, bool DR, int RB>
__device__ __forceinline__ void load_w(WRegs<RB, NG>& R, const int (&sl)[RB], const WSrc& src, int Kt, int Nb,
                                       int rbw, int kt, uint32_t vcode, uint32_t vscale, uint32_t vrs) {
  const int ktc = min(kt, Kt - 1);
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int rb = min(rbw + j, Nb - 1);
    const int tofs = (rb * Kt + ktc) * kTileBytes;
    const auto c = __builtin_amdgcn_raw_buffer_load_b128(src.tiles, vcode, tofs, 0);
    R.code[j] = make_uint4(c[0], c[1], c[2], c[3]);
    // scale rows are padded to 8 halves, so these dwords are aligned and in the row
    const int srow = rb * kRowsPerBlock * (int)src.sstride_b;
    if constexpr (NG == 1) {
      R.sraw[j] = __builtin_amdgcn_raw_buffer_load_b32(src.scales, vscale, srow + 4 * (ktc >> 1), 0);
    } else if constexpr (NG == 2) {
      R.sraw[j] = __builtin_amdgcn_raw_buffer_load_b32(src.scales, vscale, srow + 4 * ktc, 0);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(src.scales, vscale, srow + 8 * ktc, 0);
      R.sraw[j] = make_uint2(v[0], v[1]);
    }
    if constexpr (DR) {
      R.slot[j] = sl[j];
      const auto rc = __builtin_amdgcn_raw_buffer_load_b128(src.rtiles, vcode, sl[j] * kTileBytes, 0);
      R.rcode[j] = make_uint4(rc[0], rc[1], rc[2], rc[3]);
      R.rsc[j] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(src.rscale, vrs, sl[j] * kRowsPerBlock * 4, 0));
    }
  }
}

// group scale gi of the tile from the loaded dword(s)
template <int NG, class T>
__device__ __forceinline__ float group_scale(const T sraw, int kt, int gi) {
  uint32_t bits;
  if constexpr (NG == 1) bits = (kt & 1) ? (sraw >> 16) : (sraw & 0xFFFFu);
  else if constexpr (NG == 2) bits = gi ? (sraw >> 16) : (sraw & 0xFFFFu);
  else bits = ((gi < 2 ? sraw.x : sraw.y) >> (16 * (gi & 1))) & 0xFFFFu;
  return h_to_f(bits);
}

__device__ __forceinline__ i32x8_t split_nibbles(uint4 d) {
  i32x8_t b;
  b[0] = (int32_t)(d.x & kNibbleBytes);
  b[1] = (int32_t)((d.x >> 4) & kNibbleBytes);
  b[2] = (int32_t)(d.y & kNibbleBytes);
  b[3] = (int32_t)((d.y >> 4) & kNibbleBytes);
  b[4] = (int32_t)(d.z & kNibbleBytes);
  b[5] = (int32_t)((d.z >> 4) & kNibbleBytes);
  b[6] = (int32_t)(d.w & kNibbleBytes);
  b[7] = (int32_t)((d.w >> 4) & kNibbleBytes);
  return b;
}

// The lane's activation operand for group gi of the tile, read from the
// staged row: dwords 2 t, 2 t + 1 hold columns 32 t + .., so group gi is
// dwords [8 gi / NG, 8 (gi + 1) / NG); the others are zero.
template <int NG>
__device__ __forceinline__ i32x8_t load_operand(const uint8_t* p, int gi) {
  if constexpr (NG == 1) {
    return *reinterpret_cast<const i32x8_t*>(p);
  } else if constexpr (NG == 2) {
    const uint4 v = reinterpret_cast<const uint4*>(p)[gi];
    i32x8_t a = {0, 0, 0, 0, 0, 0, 0, 0};
    a[4 * gi + 0] = (int32_t)v.x;
    a[4 * gi + 1] = (int32_t)v.y;
    a[4 * gi + 2] = (int32_t)v.z;
    a[4 * gi + 3] = (int32_t)v.w;
    return a;
  } else {
    const uint2 v = reinterpret_cast<const uint2*>(p)[gi];
    i32x8_t a = {0, 0, 0, 0, 0, 0, 0, 0};
    a[2 * gi + 0] = (int32_t)v.x;
    a[2 * gi + 1] = (int32_t)v.y;
    return a;
  }
}

__device__ __forceinline__ float4_t mfma_fp8(i32x8_t a, i32x8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kE8m0One, 0, kE8m0One);
}

// The MFMAs and scalings are pure, so instruction selection may place them
// after later loads and barriers, next to the following tile's work: both
// tiles' operands would then be live at once. An opaque use of the
// accumulators (it emits no instruction) pins the math before that point.
template <int MS, int RB>
__device__ __forceinline__ void pin_acc(float4_t (&acc)[MS][RB]) {
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < RB; ++j) asm volatile("" : "+v"(acc[i][j]));
}

// One code tile: the wave's MS x RB output blocks of 16 x 16 (tokens x
// features). Lane l feeds token / feature l % 16 and k bytes 32 (l / 16) ..
// + 31 of both operands, and receives D[4 (l / 16) + 0..3][l % 16].
template <class C, int NG, bool DR>
__device__ __forceinline__ void tile_math(float4_t (&acc)[C::kMs][C::kRb], const WRegs<C::kRb, NG>& R, int kt,
                                          const uint8_t* st, int wm, int lane, int nblk) {
  constexpr int MS = C::kMs, RB = C::kRb, BM = C::kBm;
  using S = StageA4<NG, BM>;
  const int r = lane & 15, g = lane >> 4;
  const float* ms = reinterpret_cast<const float*>(st + S::kScaleOff);
  const float* mc = reinterpret_cast<const float*>(st + S::kCOff);
  i32x8_t b[RB];
  float sw[RB][NG];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    b[j] = split_nibbles(R.code[j]);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) sw[j][gi] = group_scale<NG>(R.sraw[j], kt, gi);
  }
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int row = 16 * (MS * wm + i);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const i32x8_t a = load_operand<NG>(st + (row + r) * kLdsRow + 32 * g, gi);
      const float4_t cv = *reinterpret_cast<const float4_t*>(mc + gi * BM + row + 4 * g);
      const float4_t sv = *reinterpret_cast<const float4_t*>(ms + gi * BM + row + 4 * g);
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const float4_t d = mfma_fp8(a, b[j], cv);
        acc[i][j] += d * (sv * sw[j][gi]);
      }
    }
  }
  if constexpr (DR) {
    pin_acc<MS, RB>(acc);
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      if (R.slot[j] == nblk) continue;   // wave-uniform
      const i32x8_t br = split_nibbles(R.rcode[j]);
      const float sr = R.rsc[j];
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int row = 16 * (MS * wm + i);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          const i32x8_t a = load_operand<NG>(st + (row + r) * kLdsRow + 32 * g, gi);
          const float4_t cv = *reinterpret_cast<const float4_t*>(mc + gi * BM + row + 4 * g);
          const float4_t sv = *reinterpret_cast<const float4_t*>(ms + gi * BM + row + 4 * g);
          const float4_t d = mfma_fp8(a, br, cv);
          acc[i][j] += d * (sv * sr);
        }
      }
      pin_acc<MS, RB>(acc);
    }
  }
}

// Activation tile kt of the workgroup's tokens: XR 16-byte chunks per thread
// (chunk c: token c / 8, bytes 16 (c % 8)) and, for threads below BM * NG,
// one metadata dword. Both through buffer resources over the workgroup's
// rows, so tokens past M read as zero (scale 0, C 0).
template <class C, int NG>
struct ActRegs {
  uint4 x[C::kXr];
  uint32_t meta;
};

template <class C, int NG>
__device__ __forceinline__ void load_act(ActRegs<C, NG>& A, __amdgpu_buffer_rsrc_t xrs, __amdgpu_buffer_rsrc_t mrs,
                                         int Kp, int ngt, int kt, int tid) {
#pragma unroll
  for (int i = 0; i < C::kXr; ++i) {
    const int c = tid + C::kThreads * i;
    const uint32_t off = (uint32_t)((c >> 3) * Kp + kt * kTileCols + 16 * (c & 7));
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
    A.x[i] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  const uint32_t moff = (uint32_t)(((tid / NG) * ngt + kt * NG + tid % NG) * 4);
  A.meta = __builtin_amdgcn_raw_buffer_load_b32(mrs, moff, 0, 0);
}

template <class C, int NG>
__device__ __forceinline__ void store_act(const ActRegs<C, NG>& A, uint8_t* st, int tid) {
  constexpr int BM = C::kBm;
  using S = StageA4<NG, BM>;
#pragma unroll
  for (int i = 0; i < C::kXr; ++i) {
    const int c = tid + C::kThreads * i;
    if (C::kChunks % C::kThreads == 0 || c < C::kChunks)
      *reinterpret_cast<uint4*>(st + (c >> 3) * kLdsRow + 16 * (c & 7)) = A.x[i];
  }
  if (tid < BM * NG) {
    const int row = tid / NG, gi = tid % NG;
    const float sx = h_to_f(A.meta & 0xFFFFu) * 512.0f;
    const float cv = (float)(int16_t)(uint16_t)(A.meta >> 16) * -0.015625f;
    reinterpret_cast<float*>(st + S::kScaleOff)[gi * BM + row] = sx;
    reinterpret_cast<float*>(st + S::kCOff)[gi * BM + row] = cv;
  }
}

// Output tile of workgroup b. The hardware deals workgroups to the 8 XCDs in
// turn; index i = xcd_index(b) makes each XCD's share a contiguous range.
// That range is walked in groups of GM token slices, feature slices outer
// and token slices inner, so the ~32 workgroups an XCD runs at once cover
// about 4 feature x 8 token slices: their weight and activation tiles are
// shared through its L2 instead of each bringing a weight slice of its own.
constexpr int kGroupM = 8;

__device__ __forceinline__ int xcd_index(int b, int T) {
  const int per = T >> 3, rem = T & 7, x = b & 7, local = b >> 3;
  return x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}
__device__ __forceinline__ void tile_of(int b, int MT, int NT, int& mt, int& nt) {
  const int i = xcd_index(b, MT * NT);
  const int per_group = kGroupM * NT;
  const int grp = i / per_group, first = grp * kGroupM;
  const int gm = min(MT - first, kGroupM);
  const int r = i - grp * per_group;
  nt = r / gm;
  mt = first + (r - nt * gm);
}

template <class C, int NG, bool DR>
__global__ __launch_bounds__(C::kThreads, C::kMinBlocks) void k_gemm_a4(WArrays warr, const uint8_t* __restrict__ xq,
                                                         const uint32_t* __restrict__ xmeta,
                                                         uint16_t* __restrict__ Y, float* __restrict__ part, int M,
                                                         int N, int Kt, int Nb, int NT, int T, int kt_per_split,
                                                         DenseA4 dr) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_a4[];
  constexpr int BM = C::kBm, RB = C::kRb, MS = C::kMs;
  using S = StageA4<NG, BM>;
  uint8_t* const st0 = lds_a4;
  uint8_t* const st1 = lds_a4 + S::kBytes;

  int mt, nt;
  tile_of(blockIdx.x, T / NT, NT, mt, nt);
  const int kt0 = blockIdx.y * kt_per_split, kt1 = min(Kt, kt0 + kt_per_split);
  const int rb0 = nt * (kBn / kRowsPerBlock), m0 = mt * BM;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, tid = threadIdx.x;
  const int wn = wave % C::kNwn, wm = wave / C::kNwn;
  const int rbw = rb0 + RB * wn;
  const int Kp = Kt * kTileCols, ngt = Kt * NG;
  const int rows = min(BM, M - m0);
  const WSrc src = make_wsrc(warr);
  const uint32_t vcode = 16u * (uint32_t)lane, vscale = (uint32_t)(lane & 15) * src.sstride_b,
                 vrs = 4u * (uint32_t)(lane & 15);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(xq + (int64_t)m0 * Kp), 0, rows * Kp, kBufferRaw);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(xmeta + (int64_t)m0 * ngt), 0, rows * ngt * 4, kBufferRaw);

  float4_t acc[MS][RB];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  // W0 / W1 hold the code tiles of the even / odd steps, refilled two tiles
  // ahead right after use; sl0 / sl1 the residual slots of their next refill.
  WRegs<RB, NG> W0, W1;
  int sl0[RB] = {}, sl1[RB] = {};
  ActRegs<C, NG> xa;
  if constexpr (DR) {
    load_slots(sl0, dr, Kt, Nb, rbw, kt0);
    load_slots(sl1, dr, Kt, Nb, rbw, kt0 + 1);
  }
  load_w<NG, DR>(W0, sl0, src, Kt, Nb, rbw, kt0, vcode, vscale, vrs);
  load_w<NG, DR>(W1, sl1, src, Kt, Nb, rbw, kt0 + 1, vcode, vscale, vrs);
  if constexpr (DR) {
    load_slots(sl0, dr, Kt, Nb, rbw, kt0 + 2);
    load_slots(sl1, dr, Kt, Nb, rbw, kt0 + 3);
  }
  load_act<C, NG>(xa, xrs, mrs, Kp, ngt, kt0, tid);
  store_act<C, NG>(xa, st0, tid);
  load_act<C, NG>(xa, xrs, mrs, Kp, ngt, kt0 + 1, tid);
  __syncthreads();

  auto step = [&](auto par, int kt) {
    constexpr int P = decltype(par)::value;
    uint8_t* const cur = P ? st1 : st0;
    uint8_t* const nxt = P ? st0 : st1;
    WRegs<RB, NG>& R = P ? W1 : W0;
    int(&sl)[RB] = P ? sl1 : sl0;
    tile_math<C, NG, DR>(acc, R, kt, cur, wm, lane, dr.nblk);
    pin_acc<MS, RB>(acc);
    store_act<C, NG>(xa, nxt, tid);
    load_act<C, NG>(xa, xrs, mrs, Kp, ngt, kt + 2, tid);
    load_w<NG, DR>(R, sl, src, Kt, Nb, rbw, kt + 2, vcode, vscale, vrs);
    if constexpr (DR) load_slots(sl, dr, Kt, Nb, rbw, kt + 4);
    __syncthreads();
  };
  int kt = kt0;
  for (; kt + 2 <= kt1; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
  }
  if (kt < kt1) step(std::integral_constant<int, 0>{}, kt);

  // Epilogue: acc[i][j][q] is token m0 + 16 (MS wm + i) + 4 (l / 16) + q,
  // feature 16 (rbw + j) + l % 16. With split-K, fp32 into this split's slice.
  const int r = lane & 15, g = lane >> 4;
  // (M N < 2^31 and the workspace is below 2^31 values: 32-bit indices)
  float* const pslice = part ? part + blockIdx.y * M * N : nullptr;
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int n = (rbw + j) * kRowsPerBlock + r;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < MS; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + 16 * (MS * wm + i) + 4 * g + q;
        if (m >= M) continue;
        if (pslice) pslice[m * N + n] = acc[i][j][q];
        else Y[m * N + n] = f32_to_h(acc[i][j][q]);
      }
    }
  }
}

// the handle's arrays for the kernels' buffer resources
template <bool DR>
WArrays weight_arrays(const mq_packed* p) {
  WArrays w;
  w.tiles = p->tiles;
  w.tiles_b = (int)(p->Nb * p->Kt * kTileBytes);
  w.scales = p->scales;
  w.scales_b = (int)(p->Nb * kRowsPerBlock * p->sstride * 2);
  w.sstride_b = (uint32_t)(p->sstride * 2);
  w.rtiles = DR ? (const void*)p->rt_tiles : (const void*)p->tiles;
  w.rtiles_b = DR ? (int)((p->nblk + 1) * kTileBytes) : 0;
  w.rscale = DR ? (const void*)p->bscale : (const void*)p->tiles;
  w.rscale_b = DR ? (int)((p->nblk + 1) * kRowsPerBlock * 4) : 0;
  return w;
}

template <class C, int NG, bool DR>
hipError_t launch_a4(const mq_packed* p, const uint8_t* xq, const uint32_t* xmeta, int64_t M, uint16_t* Y,
                     hipStream_t s) {
  constexpr int BM = C::kBm;
  constexpr size_t kLds = 2 * (size_t)StageA4<NG, BM>::kBytes;
  static bool attr_set = false;
  if (!attr_set && kLds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_a4<C, NG, DR>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int NT = (int)((p->Nb + 15) / 16);
  const int MT = (int)((M + BM - 1) / BM);
  const int T = NT * MT;
  const int Kt = (int)p->Kt;
  int S = 1;
  if (T < kSplitTarget) S = std::max(1, std::min(kSplitTarget / T, Kt / 2));
  const int per = (Kt + S - 1) / S;
  S = (Kt + per - 1) / per;
  float* part = nullptr;
  if (S > 1) {
    const hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&part), (size_t)S * M * p->N * sizeof(float), s);
    if (e != hipSuccess) return e;
  }
  const DenseA4 dr = DR ? DenseA4{p->rt_slot, reinterpret_cast<const uint4*>(p->rt_tiles), p->bscale, (int)p->nblk}
                        : DenseA4{nullptr, nullptr, nullptr, 0};
  const WArrays warr = weight_arrays<DR>(p);
  k_gemm_a4<C, NG, DR><<<dim3((unsigned)T, (unsigned)S), dim3(C::kThreads), kLds, s>>>(
      warr, xq, xmeta, Y, part, (int)M, (int)p->N, Kt, (int)p->Nb, NT, T, per, dr);
  hipError_t e = hipGetLastError();
  if (S > 1) {
    if (e == hipSuccess) e = launch_splitk_reduce(part, Y, M, p->N, S, s);
    const hipError_t f = hipFreeAsync(part, s);
    if (e == hipSuccess) e = f;
  }
  return e;
}

template <class C, bool DR>
hipError_t launch_a4_g(const mq_packed* p, const uint8_t* xq, const uint32_t* xmeta, int64_t M, uint16_t* Y,
                       hipStream_t s) {
  if (p->G == 128) return launch_a4<C, 1, DR>(p, xq, xmeta, M, Y, s);
  if (p->G == 64) return launch_a4<C, 2, DR>(p, xq, xmeta, M, Y, s);
  return launch_a4<C, 4, DR>(p, xq, xmeta, M, Y, s);
}

template <class C>
hipError_t launch_a4_d(const mq_packed* p, const uint8_t* xq, const uint32_t* xmeta, int64_t M, uint16_t* Y,
                       hipStream_t s) {
  return (p->blocks && p->nblk > 0) ? launch_a4_g<C, true>(p, xq, xmeta, M, Y, s)
                                    : launch_a4_g<C, false>(p, xq, xmeta, M, Y, s);
}

// ------------------------------------------------------------- W4A4 decode

// Decode (M <= 16): one workgroup per RBW row blocks with the full K; its 8
// waves split the column tiles, so no partial sums leave the workgroup (no
// workspace, no second kernel). Each wave requests the codes, scales and
// residual tiles of up to 4 of its tiles (2 when G < 128) for all RBW row
// blocks, and their
// activation codes and metadata, before any math; the 8 partial sums of
// each row block meet in LDS and are added in wave order.
template <int NG>
constexpr int dec_tiles() { return NG == 1 ? 4 : 2; }   // tiles a wave loads ahead (fewer registers for G < 128)
constexpr int64_t kDecMaxM = 16;   // tokens of one 16-row MFMA operand

template <int NG, int RBW>
struct DecRegs {
  static constexpr int T = dec_tiles<NG>();
  uint4 code[T][RBW];
  typename WRegs<RBW, NG>::SrawT sraw[T][RBW];
  uint4 rcode[T][RBW];
  float rsc[T][RBW];
  int slot[T][RBW];
  uint4 a0[T], a1[T];        // the lane's 32 activation bytes (token l % 16) of each tile
  uint32_t meta[T][4][NG];   // metadata of tokens 4 (l / 16) + 0..3 of each tile
};

// Activations quantized inside the decode kernel (QX): up to kDecQxMaxM
// tokens and K <= kDecQxMaxK, held in LDS in the layout of the quantizer's
// output.
constexpr int kDecQxMaxM = 2;
constexpr int kDecQxMaxK = 4096;

// The lane's activation operand and metadata of tile kt (tokens past M read
// zero codes and metadata): from the quantizer's output in global memory, or
// with QX from its copy in LDS.
template <int NG, bool QX>
__device__ __forceinline__ void dec_load_x(uint4& a0, uint4& a1, uint32_t (&meta)[4][NG],
                                           __amdgpu_buffer_rsrc_t xrs, __amdgpu_buffer_rsrc_t mrs,
                                           const uint8_t* xq_s, const uint32_t* meta_s, int M, int Kp, int ngt,
                                           uint32_t va, int r, int g, int kt) {
  if constexpr (QX) {
    const int rr = min(r, M - 1);   // a token past M repeats the last one; its outputs are never stored
    const uint4* p = reinterpret_cast<const uint4*>(xq_s + rr * Kp + kt * kTileCols + 32 * g);
    a0 = p[0];
    a1 = p[1];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) meta[q][gi] = meta_s[min(4 * g + q, M - 1) * ngt + kt * NG + gi];
  } else {
    const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(xrs, va, kt * kTileCols, 0);
    const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(xrs, va, kt * kTileCols + 16, 0);
    a0 = make_uint4(v0[0], v0[1], v0[2], v0[3]);
    a1 = make_uint4(v1[0], v1[1], v1[2], v1[3]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
        meta[q][gi] = __builtin_amdgcn_raw_buffer_load_b32(mrs, (uint32_t)(((4 * g + q) * ngt + kt * NG + gi) * 4), 0, 0);
  }
}

// The weight side of tile kt for the RBW row blocks: codes, scales, and the
// block residual's tile and row scale.
template <int NG, bool DR, int RBW>
__device__ __forceinline__ void dec_load_w(DecRegs<NG, RBW>& D, int t, const WSrc& src, const DenseA4& dr,
                                           int rb0, int Nb, int Kt, int kt, uint32_t vcode, uint32_t vscale,
                                           uint32_t vrs) {
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    const int rb = min(rb0 + j, Nb - 1);
    const auto c = __builtin_amdgcn_raw_buffer_load_b128(src.tiles, vcode, (rb * Kt + kt) * kTileBytes, 0);
    D.code[t][j] = make_uint4(c[0], c[1], c[2], c[3]);
    const int srow = rb * kRowsPerBlock * (int)src.sstride_b;
    if constexpr (NG == 1) {
      D.sraw[t][j] = __builtin_amdgcn_raw_buffer_load_b32(src.scales, vscale, srow + 4 * (kt >> 1), 0);
    } else if constexpr (NG == 2) {
      D.sraw[t][j] = __builtin_amdgcn_raw_buffer_load_b32(src.scales, vscale, srow + 4 * kt, 0);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(src.scales, vscale, srow + 8 * kt, 0);
      D.sraw[t][j] = make_uint2(v[0], v[1]);
    }
    if constexpr (DR) {
      const int sl = __builtin_amdgcn_readfirstlane(dr.slot[(int64_t)rb * Kt + kt]);
      D.slot[t][j] = sl;
      const auto rc = __builtin_amdgcn_raw_buffer_load_b128(src.rtiles, vcode, sl * kTileBytes, 0);
      D.rcode[t][j] = make_uint4(rc[0], rc[1], rc[2], rc[3]);
      D.rsc[t][j] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(src.rscale, vrs, sl * kRowsPerBlock * 4, 0));
    }
  }
}

// QX: the workgroup's 512 threads quantize the M token rows (every tile)
// into LDS, 16 lanes per (token, tile) as in the quantizer kernel, in two
// parts: the loads of the thread's PQ chunks (issued before the weight
// loads, so that waiting for them waits for nothing else; chunks past the
// batch or past K read zero through the buffer's range), then the
// quantization into LDS.
template <int PQ>
__device__ __forceinline__ void dec_quant_load(uint4 (&xv)[PQ], __amdgpu_buffer_rsrc_t xs, int K, int Kt, int units) {
#pragma unroll
  for (int i = 0; i < PQ; ++i) {
    const int u = (int)threadIdx.x + 512 * i;
    const int pair = u >> 4, c = u & 15;
    const int m = pair / Kt, kt = pair - m * Kt;
    const int col0 = 128 * kt + 32 * (c & 3) + 8 * (c >> 2);
    const uint32_t off = (u < units && col0 < K) ? (uint32_t)(m * K + col0) * 2u : 0x7FFFFFF0u;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(xs, off, 0, 0);
    xv[i] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

template <int NG, int PQ>
__device__ __forceinline__ void dec_quant_store(const uint4 (&xv)[PQ], int Kt, int units, uint8_t* xq_s,
                                                uint32_t* meta_s) {
  const int Kp = Kt * kTileCols;
#pragma unroll
  for (int i = 0; i < PQ; ++i) {
    const int u = (int)threadIdx.x + 512 * i;
    if (u < units) {   // units is a multiple of 16: a 16-lane group is all in or all out
      const int pair = u >> 4, c = u & 15;
      const int m = pair / Kt, kt = pair - m * Kt;
      quant_chunk_v<NG>(xv[i], c, xq_s + m * Kp + 128 * kt, meta_s + (m * Kt + kt) * NG);
    }
  }
  // publish the codes: an LDS-only barrier (the weight loads stay in flight)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int NG, bool DR, int RBW, bool QX, int PQ>
__global__ __launch_bounds__(512) void k_gemv_a4(WArrays warr, const uint8_t* __restrict__ xq,
                                                 const uint32_t* __restrict__ xmeta, const uint16_t* __restrict__ X,
                                                 int K, uint16_t* __restrict__ Y, int M, int N, int Kt, int Nb,
                                                 DenseA4 dr) {
  __shared__ float4_t red[RBW][8][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int rb0 = blockIdx.x * RBW;
  const int kt0 = (Kt * wave) / 8, kt1 = (Kt * (wave + 1)) / 8;
  const WSrc src = make_wsrc(warr);
  const int Kp = Kt * kTileCols, ngt = Kt * NG;
  // tokens past M read as zero codes and zero metadata
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(xq), 0, QX ? 0 : M * Kp, kBufferRaw);
  const __amdgpu_buffer_rsrc_t mrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(xmeta), 0, QX ? 0 : M * ngt * 4, kBufferRaw);
  const uint32_t vcode = 16u * (uint32_t)lane, vscale = (uint32_t)r * src.sstride_b, vrs = 4u * (uint32_t)r;
  const uint32_t va = (uint32_t)(r * Kp + 32 * g);
  uint8_t* xq_s = nullptr;
  uint32_t* meta_s = nullptr;
  if constexpr (QX) {
    __shared__ __attribute__((aligned(16))) uint8_t xq_lds[kDecQxMaxM * kDecQxMaxK];
    __shared__ uint32_t meta_lds[kDecQxMaxM * (kDecQxMaxK / 32)];
    xq_s = xq_lds;
    meta_s = meta_lds;
  }

  float4_t acc[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int units = M * Kt * 16;
  uint4 xv[QX ? PQ : 1];
  if constexpr (QX) {
    const __amdgpu_buffer_rsrc_t xs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), 0, M * K * 2, kBufferRaw);
    dec_quant_load<PQ>(xv, xs, K, Kt, units);
    // memory operations keep their program order across this point (no
    // register is named, so nothing waits here): the X loads go out first
    asm volatile("" ::: "memory");
  }

  constexpr int T = dec_tiles<NG>();
  bool first = true;
  for (int base = kt0; base < kt1; base += T) {
    DecRegs<NG, RBW> D;
    // every load of the batch first (tiles past kt1 are clamped; their math is skipped)
    if constexpr (QX) {
      // the weight loads go out first; the first batch's are in flight while
      // the workgroup quantizes the activations into LDS
#pragma unroll
      for (int t = 0; t < T; ++t) dec_load_w<NG, DR, RBW>(D, t, src, dr, rb0, Nb, Kt, min(base + t, Kt - 1), vcode, vscale, vrs);
      if (first) {
        // The quantization starts only here, after the weight requests: the
        // empty asm redefines the X registers (and orders memory), so none
        // of the arithmetic can move above it, and the wait it needs covers
        // the X loads alone (issued first; the weight loads stay in flight).
#pragma unroll
        for (int i = 0; i < PQ; ++i)
          asm volatile("" : "+v"(xv[i].x), "+v"(xv[i].y), "+v"(xv[i].z), "+v"(xv[i].w) :: "memory");
        dec_quant_store<NG, PQ>(xv, Kt, units, xq_s, meta_s);
        first = false;
      }
#pragma unroll
      for (int t = 0; t < T; ++t)
        dec_load_x<NG, true>(D.a0[t], D.a1[t], D.meta[t], xrs, mrs, xq_s, meta_s, M, Kp, ngt, va, r, g,
                             min(base + t, Kt - 1));
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int kt = min(base + t, Kt - 1);
        dec_load_x<NG, false>(D.a0[t], D.a1[t], D.meta[t], xrs, mrs, xq_s, meta_s, M, Kp, ngt, va, r, g, kt);
        dec_load_w<NG, DR, RBW>(D, t, src, dr, rb0, Nb, Kt, kt, vcode, vscale, vrs);
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int kt = base + t;
      if (kt >= kt1) break;   // wave-uniform
      i32x8_t a;
      a[0] = (int32_t)D.a0[t].x; a[1] = (int32_t)D.a0[t].y; a[2] = (int32_t)D.a0[t].z; a[3] = (int32_t)D.a0[t].w;
      a[4] = (int32_t)D.a1[t].x; a[5] = (int32_t)D.a1[t].y; a[6] = (int32_t)D.a1[t].z; a[7] = (int32_t)D.a1[t].w;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        i32x8_t ag = a;
        if constexpr (NG > 1) {
          constexpr int W = 8 / NG;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (k / W != gi) ag[k] = 0;
        }
        float4_t cv, sv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t mv = D.meta[t][q][gi];
          sv[q] = h_to_f(mv & 0xFFFFu) * 512.0f;
          cv[q] = (float)(int16_t)(uint16_t)(mv >> 16) * -0.015625f;
        }
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
          const float sw = group_scale<NG>(D.sraw[t][j], kt, gi);
          const float4_t d = mfma_fp8(ag, split_nibbles(D.code[t][j]), cv);
          acc[j] += d * (sv * sw);
          if constexpr (DR) {
            if (D.slot[t][j] != dr.nblk) {   // wave-uniform
              const float4_t e = mfma_fp8(ag, split_nibbles(D.rcode[t][j]), cv);
              acc[j] += e * (sv * D.rsc[t][j]);
            }
          }
        }
      }
    }
  }
  if constexpr (QX) {
    if (first) dec_quant_store<NG, PQ>(xv, Kt, units, xq_s, meta_s);   // a wave with no tiles (Kt < 8)
  }

#pragma unroll
  for (int j = 0; j < RBW; ++j) red[j][wave][lane] = acc[j];
  __syncthreads();
  if (wave < RBW && rb0 + wave < Nb) {   // wave j adds row block j's 8 partials in wave order
    float4_t sum = red[wave][0][lane];
#pragma unroll
    for (int w = 1; w < 8; ++w) sum += red[wave][w][lane];
    const int n = (rb0 + wave) * kRowsPerBlock + r;
    if (n < N) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 4 * g + q;
        if (m < M) Y[m * N + n] = f32_to_h(sum[q]);
      }
    }
  }
}

// QX: X holds the fp16 activations (K columns), quantized inside the kernel;
// otherwise xq / xmeta hold the quantizer's output.
template <int NG, bool DR, int RBW, bool QX>
hipError_t launch_dec(const mq_packed* p, const uint8_t* xq, const uint32_t* xmeta, const uint16_t* X, int64_t M,
                      uint16_t* Y, hipStream_t s) {
  const WArrays warr = weight_arrays<DR>(p);
  const DenseA4 dr = DR ? DenseA4{p->rt_slot, reinterpret_cast<const uint4*>(p->rt_tiles), p->bscale, (int)p->nblk}
                        : DenseA4{nullptr, nullptr, nullptr, 0};
  const unsigned grid = (unsigned)((p->Nb + RBW - 1) / RBW);
  // QX: 16 M Kt / 512 <= 2 chunks per thread (M <= 2, Kt <= 32)
  constexpr int PQ = QX ? (16 * kDecQxMaxM * (kDecQxMaxK / kTileCols)) / 512 : 1;
  k_gemv_a4<NG, DR, RBW, QX, PQ><<<dim3(grid), dim3(512), 0, s>>>(warr, xq, xmeta, X, (int)p->K, Y, (int)M,
                                                                 (int)p->N, (int)p->Kt, (int)p->Nb, dr);
  return hipGetLastError();
}

// row blocks per workgroup: enough that one round of workgroups covers the
// layer on 256 CUs, at most 4
template <int NG, bool DR, bool QX>
hipError_t launch_dec_r(const mq_packed* p, const uint8_t* xq, const uint32_t* xmeta, const uint16_t* X, int64_t M,
                        uint16_t* Y, hipStream_t s) {
  const int64_t rbw = std::min<int64_t>(4, std::max<int64_t>(1, (p->Nb + 255) / 256));
  if (rbw == 1) return launch_dec<NG, DR, 1, QX>(p, xq, xmeta, X, M, Y, s);
  if (rbw == 2) return launch_dec<NG, DR, 2, QX>(p, xq, xmeta, X, M, Y, s);
  if (rbw == 3) return launch_dec<NG, DR, 3, QX>(p, xq, xmeta, X, M, Y, s);
  return launch_dec<NG, DR, 4, QX>(p, xq, xmeta, X, M, Y, s);
}

template <bool DR, bool QX>
hipError_t launch_dec_g(const mq_packed* p, const uint8_t* xq, const uint32_t* xmeta, const uint16_t* X, int64_t M,
                        uint16_t* Y, hipStream_t s) {
  if (p->G == 128) return launch_dec_r<1, DR, QX>(p, xq, xmeta, X, M, Y, s);
  if (p->G == 64) return launch_dec_r<2, DR, QX>(p, xq, xmeta, X, M, Y, s);
  return launch_dec_r<4, DR, QX>(p, xq, xmeta, X, M, Y, s);
}

}  // namespace

hipError_t quantize_a4(const uint16_t* X, int64_t M, int64_t K, int G, uint8_t* xq, uint32_t* xmeta, hipStream_t s) {
  const int Kt = (int)((K + kTileCols - 1) / kTileCols);
  const int64_t threads = M * Kt * 16;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (G == 128) k_quant_a4<1><<<grid, block, 0, s>>>(X, (int)M, (int)K, Kt, xq, xmeta);
  else if (G == 64) k_quant_a4<2><<<grid, block, 0, s>>>(X, (int)M, (int)K, Kt, xq, xmeta);
  else k_quant_a4<4><<<grid, block, 0, s>>>(X, (int)M, (int)K, Kt, xq, xmeta);
  return hipGetLastError();
}

hipError_t launch_gemm_a4(const mq_packed* p, const uint8_t* xq, const uint32_t* xmeta, int64_t M, uint16_t* Y,
                          hipStream_t s) {
  if (M <= kDecMaxM) {
    return (p->blocks && p->nblk > 0) ? launch_dec_g<true, false>(p, xq, xmeta, nullptr, M, Y, s)
                                      : launch_dec_g<false, false>(p, xq, xmeta, nullptr, M, Y, s);
  }
  return launch_a4_d<CfgA4Mid>(p, xq, xmeta, M, Y, s);
}

bool decode_a4_fused_takes(const mq_packed* p, int64_t M) {
  return M >= 1 && M <= kDecQxMaxM && p->K <= kDecQxMaxK;
}

hipError_t launch_decode_a4_fused(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  return (p->blocks && p->nblk > 0) ? launch_dec_g<true, true>(p, nullptr, nullptr, X, M, Y, s)
                                    : launch_dec_g<false, true>(p, nullptr, nullptr, X, M, Y, s);
}

}  // namespace mq
