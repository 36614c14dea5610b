// Device helpers shared by the two fused kernels (decode GEMV and prefill GEMM).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace mq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Buffer descriptor word 3 for raw (unswizzled) byte addressing with a 32-bit
// data format: loads past the descriptor's byte range return zero.
constexpr int kBufferRaw = 0x00020000;

// D = (a & m) | o, one v_and_or_b32 when m and o already sit in VGPRs (a
// VOP3 instruction on this target takes at most one scalar operand). Plain C
// rather than inline asm: the compiler's hazard checks do not see into an asm
// block, and a VGPR written by one while an MFMA still reads it as its
// accumulator input would corrupt that MFMA.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) { return (a & m) | o; }

// The 8 codes of one dword as exact fp16 q = u - 8 (no scale). Pairs (0,1)
// and (4,5) sit in nibbles 0/4 of the dword and of the dword shifted right
// by 8: masked with 0x000F000F into fp16 1024.0 they give 1024 + u, and
// (1024 + u) - 1032 = q. Pairs (2,3) and (6,7) are masked in place with
// 0x00F000F0, giving 1024 + 16 u, and (1024 + 16 u) / 16 - 72 = q in one
// fused multiply-add (every value is exact in fp16). 9 VALU ops for 8 codes.
// vmask = 0x000F000F, vmask4 = 0x00F000F0, vmagic = 0x64006400 in VGPRs.
__device__ __forceinline__ half8_t widen_q(uint32_t w, uint32_t vmask, uint32_t vmask4, uint32_t vmagic) {
  const half2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t k72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w8 = w >> 8;
  u32x4_t v;
  v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, and_or(w, vmask, vmagic)) - bias);
  v.y = __builtin_bit_cast(uint32_t,
                           __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(w, vmask4, vmagic)), k16, k72));
  v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, and_or(w8, vmask, vmagic)) - bias);
  v.w = __builtin_bit_cast(uint32_t,
                           __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(w8, vmask4, vmagic)), k16, k72));
  return __builtin_bit_cast(half8_t, v);
}

// The 8 codes of one dword as fp16(s q): exact q as in widen_q, then one
// packed multiply by the group scale (a single rounding of s q).
__device__ __forceinline__ half8_t dequant_dword(uint32_t w, half2_t s2, uint32_t vmask, uint32_t vmask4,
                                                 uint32_t vmagic) {
  // (vector elements are copied to scalars first: a bit_cast of an element
  // lvalue such as v.y reads element 0 with this compiler)
  const u32x4_t q = __builtin_bit_cast(u32x4_t, widen_q(w, vmask, vmask4, vmagic));
  const uint32_t q0 = q.x, q1 = q.y, q2 = q.z, q3 = q.w;
  u32x4_t v;
  v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q0) * s2);
  v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q1) * s2);
  v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q2) * s2);
  v.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q3) * s2);
  return __builtin_bit_cast(half8_t, v);
}

__device__ __forceinline__ float h_to_f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ half2_t splat_half(uint32_t bits16) {
  return __builtin_bit_cast(half2_t, bits16 | (bits16 << 16));
}

__device__ __forceinline__ half8_t as_half8(uint4 v) {
  u32x4_t u;
  u.x = v.x;
  u.y = v.y;
  u.z = v.z;
  u.w = v.w;
  return __builtin_bit_cast(half8_t, u);
}

// D += A B on a 16x16x32 fp16 MFMA with fp32 accumulation. Lane l supplies
// A[l % 16][8 (l / 16) + 0..7] and B[8 (l / 16) + 0..7][l % 16], and receives
// D[4 (l / 16) + 0..3][l % 16].
__device__ __forceinline__ float4_t mfma16(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Residual stream entry: column mod 4096 | row mod 16 | fp16 residual value sr*qr.
__device__ __forceinline__ uint32_t ent_col(uint32_t e) { return e & 0xFFFu; }
__device__ __forceinline__ uint32_t ent_row(uint32_t e) { return (e >> 12) & 15u; }
__device__ __forceinline__ uint32_t ent_delta(uint32_t e) { return e >> 16; }

// Tile index of workgroup b: the hardware deals workgroups to the 8 XCDs in
// turn, so the tiles of XCD x are made a contiguous range (one or a few
// token slices, all their feature tiles).
__device__ __forceinline__ int xcd_tile(int b, int T) {
  const int per = T >> 3, rem = T & 7, x = b & 7, local = b >> 3;
  return x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}

// X of one token block (16 token rows) for one code tile (128 columns) as a
// 4 KiB LDS block in the B-operand order of the 16x16x32 fp16 MFMA, filled
// by 4 loads of 64 lanes x 16 bytes written in lane order (registers stored
// in lane order, or direct copies into LDS): lane l = 16 a + j of load u
// reads 8 columns of token row 4 u + a, chunk 4 ((j / 4) ^ u) + ((j % 4) ^ a)
// of the tile's 16 chunks of 8 columns. The 4 lanes of a quad read one
// 64-byte run (loading the B order directly would have each quad read 4
// token rows, which the L2-to-CU path serves at well under half the rate),
// and the loads put token row c, chunk h at 16-byte position
// 64 (c / 4) + 16 (c % 4) + 4 ((h / 4) ^ (c / 4)) + ((h % 4) ^ (c % 4)).
// The B operand of k-step t in lane n + 16 g is row n, chunk 4 t + g; for
// fixed t and g the 16 lanes n read 16 distinct 16-byte bank groups.
__device__ __forceinline__ uint32_t x_load_chunk(int lane, int u) {
  return 4u * (uint32_t)(((lane & 15) >> 2) ^ u) + (uint32_t)((lane & 3) ^ (lane >> 4));
}
__device__ __forceinline__ uint32_t x_read_pos(int lane, int t) {
  const int n = lane & 15, g = lane >> 4;
  return (uint32_t)(64 * (n >> 2) + 16 * (n & 3) + 4 * (t ^ (n >> 2)) + (g ^ (n & 3)));
}

// fp32 -> fp16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Store 4 consecutive outputs (as fp16) of which the first `valid` exist; one
// 8-byte store when all 4 exist and the row is 8-byte aligned.
__device__ __forceinline__ void store4(uint16_t* y, float4_t s, int valid, bool aligned) {
  if (valid >= 4 && aligned) {
    const uint32_t lo = (uint32_t)f32_to_h(s.x) | ((uint32_t)f32_to_h(s.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_h(s.z) | ((uint32_t)f32_to_h(s.w) << 16);
    *reinterpret_cast<uint2*>(y) = make_uint2(lo, hi);
  } else {
    if (valid > 0) y[0] = f32_to_h(s.x);
    if (valid > 1) y[1] = f32_to_h(s.y);
    if (valid > 2) y[2] = f32_to_h(s.z);
    if (valid > 3) y[3] = f32_to_h(s.w);
  }
}

}  // namespace mq
