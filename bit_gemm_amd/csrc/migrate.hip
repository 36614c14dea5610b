// Moving activation outliers into the weights before packing, on the GPU.
//
// MosaicQuant explainer, Methodology section 1: the method first migrates
// activation outliers into the weight matrix with an equivalent
// transformation (SmoothQuant or QuaRot), then decomposes the migrated
// matrix. Here the SmoothQuant form at strength 1/2 with power-of-two
// factors: input channel j is scaled by 2^e_j in W and by 2^-e_j in X, so
// X W^T is unchanged and both scalings are exact in fp16 (one round-half-even
// rounding where a value falls below the normal range).
//   e_j = floor((E_x - E_w) / 2), E = floor(log2 max |.|) of channel j (from
//   the float's exponent, integers only); 0 when either maximum is 0; clamped
//   so that neither scaled maximum leaves fp16's range (exponent <= 15) and
//   to [-24, 24].
// Kernels: k_col_amax (per-column max |w| as fp16 magnitude bits, vector
// atomic max: order-free), k_smooth_exp (the exponents), k_scale_cols
// (A_ij 2^e_j rounded once to fp16; used for W with e and for X with -e).
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int kFp16MaxExp = 15;
constexpr int kExpClamp = 24;
constexpr uint32_t kFlagBadAmax = 1u;

// floor(log2 |v|) of a nonzero fp16 magnitude bit pattern (exact)
__device__ __forceinline__ int floor_log2_fp16(uint32_t h) {
  const int e5 = (int)((h >> 10) & 31u);
  if (e5 == 0) return (31 - __builtin_clz(h & 1023u)) - 24;   // subnormal: m 2^-24
  return e5 - 15;
}

// floor(log2 v) of a positive finite fp32 bit pattern (exact)
__device__ __forceinline__ int floor_log2_fp32(uint32_t b) {
  const int e8 = (int)((b >> 23) & 255u);
  if (e8 == 0) return (31 - __builtin_clz(b & 0x7FFFFFu)) - 149;   // subnormal: m 2^-149
  return e8 - 127;
}

// rows are dealt to the grid's y dimension in slabs; each thread keeps the
// max over its slab of one column, then one atomic max per slab
__global__ __launch_bounds__(256) void k_col_amax(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                  int rows_per_slab, uint32_t* __restrict__ amax) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= K) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_slab, r1 = min(N, r0 + rows_per_slab);
  uint32_t m = 0;
  for (int64_t i = r0; i < r1; ++i) m = max(m, (uint32_t)W[i * K + j] & 0x7FFFu);
  if (m) atomicMax(&amax[j], m);
}

__global__ __launch_bounds__(256) void k_smooth_exp(const uint32_t* __restrict__ amax_w,
                                                    const float* __restrict__ amax_x, int64_t K,
                                                    int32_t* __restrict__ e_out, uint32_t* __restrict__ flags) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= K) return;
  const float ax = amax_x[j];
  if (!(ax >= 0.0f && ax <= 3.4028234663852886e38f)) atomicOr(flags, kFlagBadAmax);   // negative, inf, NaN
  const uint32_t hw = amax_w[j];
  int e = 0;
  if (hw != 0u && ax > 0.0f) {
    const int Ew = floor_log2_fp16(hw), Ex = floor_log2_fp32(__builtin_bit_cast(uint32_t, ax));
    e = (Ex - Ew) >> 1;                                  // floor of the half difference
    const int hi = min(kFp16MaxExp - Ew, kExpClamp), lo = max(Ex - kFp16MaxExp, -kExpClamp);
    e = min(max(e, lo), hi);
  }
  e_out[j] = e;
}

// out_ij = fp16(in_ij 2^(sign e_j)): the product is exact in fp32, one rounding to fp16
__global__ __launch_bounds__(256) void k_scale_cols(const uint16_t* __restrict__ in, int64_t rows, int64_t K,
                                                    const int32_t* __restrict__ e, int sign,
                                                    uint16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * K) return;
  const int64_t j = idx % K;
  const float v = (float)__builtin_bit_cast(_Float16, in[idx]);
  out[idx] = __builtin_bit_cast(uint16_t, (_Float16)ldexpf(v, sign * e[j]));
}

}  // namespace

hipError_t smooth_weights(const uint16_t* W, int64_t N, int64_t K, const float* amax_x, uint16_t* W_out,
                          int32_t* e_out, hipStream_t s, uint32_t* flags_out) {
  uint32_t* buf = nullptr;   // [K] column maxima, then 1 flag word
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&buf), (size_t)(K + 1) * sizeof(uint32_t));
  if (e != hipSuccess) return e;
  e = hipMemsetAsync(buf, 0, (size_t)(K + 1) * sizeof(uint32_t), s);
  const int slab = 256;
  const unsigned gx = (unsigned)((K + 255) / 256), gy = (unsigned)((N + slab - 1) / slab);
  if (e == hipSuccess) {
    k_col_amax<<<dim3(gx, gy), dim3(256), 0, s>>>(W, N, K, slab, buf);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    k_smooth_exp<<<dim3(gx), dim3(256), 0, s>>>(buf, amax_x, K, e_out, buf + K);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    k_scale_cols<<<dim3((unsigned)((N * K + 255) / 256)), dim3(256), 0, s>>>(W, N, K, e_out, 1, W_out);
    e = hipGetLastError();
  }
  uint32_t flags = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&flags, buf + K, sizeof(flags), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(buf);
  *flags_out = flags;
  return e;
}

hipError_t smooth_activations(const uint16_t* X, int64_t M, int64_t K, const int32_t* e, uint16_t* X_out,
                              hipStream_t s) {
  k_scale_cols<<<dim3((unsigned)((M * K + 255) / 256)), dim3(256), 0, s>>>(X, M, K, e, -1, X_out);
  return hipGetLastError();
}

}  // namespace mq
