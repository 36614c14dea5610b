// Device helpers shared by the two fused kernels (decode GEMV and prefill GEMM).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace mq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One dword of the tile layout holds 8 codes u = q + 8 of columns c0..c0+7,
// column c in nibble (c / 2) + 4 (c % 2). OR-ing a nibble into the mantissa of
// fp16 1024.0 (0x6400) gives exactly 1024 + u, so (1024 + u) - 1032 = q exactly
// and one fp16 multiply by the group scale gives fp16(s q), correctly rounded.
__device__ __forceinline__ half8_t dequant_dword(uint32_t w, half2_t s2) {
  constexpr uint32_t kMagic = 0x64006400u;
  const half2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  const uint32_t p0 = (w & 0x000F000Fu) | kMagic;
  const uint32_t p1 = ((w >> 4) & 0x000F000Fu) | kMagic;
  const uint32_t p2 = ((w >> 8) & 0x000F000Fu) | kMagic;
  const uint32_t p3 = ((w >> 12) & 0x000F000Fu) | kMagic;
  const half2_t h0 = (__builtin_bit_cast(half2_t, p0) - bias) * s2;
  const half2_t h1 = (__builtin_bit_cast(half2_t, p1) - bias) * s2;
  const half2_t h2 = (__builtin_bit_cast(half2_t, p2) - bias) * s2;
  const half2_t h3 = (__builtin_bit_cast(half2_t, p3) - bias) * s2;
  u32x4_t v;
  v.x = __builtin_bit_cast(uint32_t, h0);
  v.y = __builtin_bit_cast(uint32_t, h1);
  v.z = __builtin_bit_cast(uint32_t, h2);
  v.w = __builtin_bit_cast(uint32_t, h3);
  return __builtin_bit_cast(half8_t, v);
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

// Residual stream entry: column mod 4096 | row mod 16 | fp16 correction.
__device__ __forceinline__ uint32_t ent_col(uint32_t e) { return e & 0xFFFu; }
__device__ __forceinline__ uint32_t ent_row(uint32_t e) { return (e >> 12) & 15u; }
__device__ __forceinline__ uint32_t ent_delta(uint32_t e) { return e >> 16; }

// fp32 -> fp16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

}  // namespace mq
