// Separate residual kernel: Y <- fp16(Y + X R^T), R the sparse residual
// (R_ij = sr_i * qr_ij on the selected entries), read from the canonical CSR.
//
// This is the unfused alternative that the pages argue against (MosaicQuant
// explainer, Methodology section 3, ZipperEngine): a dense 4-bit kernel
// followed by a second sparse kernel, which has to load the activations
// again and merge its partial output into Y. Run after mq_linear on a
// residual-free packing of the same weights it gives the unfused result, so
// the cost of not fusing can be measured. It is meant for the decode regime.
//
// A workgroup (8 waves) owns a range of rows and a chunk of TC <= 64 tokens:
// it copies X[m0 .. m0 + TC) into LDS once.
// Each wave then takes its rows one at a time: lane l holds entry l of the
// row (rows longer than 64 entries take more passes); for each token the
// wave sums qr * x over its lanes in a fixed order (DPP steps and four lane
// reads, no LDS), lane t keeps token t's sum and adds sr * sum to Y. The next
// row's bounds, first 64 entries and Y values are loaded while the current
// row computes, so the wave does not wait on memory per row. Rows without
// entries are not touched.
#include <algorithm>

#include "kernel_common.h"
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int kResThreads = 512;
constexpr int kResLdsBytes = 160 * 1024;   // the whole LDS of a CU

// Sum of v over the 64 lanes, the same in every lane, in a fixed order: DPP
// steps give every lane its 16-lane row sum (pairs, quads, 8-lane halves,
// rows), then the four row sums are read out of lanes 0, 16, 32 and 48.
template <int CTRL>
__device__ __forceinline__ float dpp_plus(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_plus<0xB1>(v);    // quad_perm [1,0,3,2]: pairs
  v = dpp_plus<0x4E>(v);    // quad_perm [2,3,0,1]: quads
  v = dpp_plus<0x141>(v);   // row_half_mirror: 8 lanes
  v = dpp_plus<0x140>(v);   // row_mirror: 16 lanes
  const int b = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

__device__ __forceinline__ void load_entry(const uint16_t* __restrict__ col, const uint8_t* __restrict__ rcodes,
                                           int e, int e1, int& c, float& q) {
  c = 0;
  q = 0.f;
  if (e < e1) {
    c = col[e];
    q = (float)((int)((rcodes[e >> 1] >> (4 * (e & 1))) & 0xFu) - 8);
  }
}

__global__ __launch_bounds__(kResThreads) void k_residual(const int32_t* __restrict__ row_ptr,
                                                          const uint16_t* __restrict__ col,
                                                          const uint8_t* __restrict__ rcodes,
                                                          const float* __restrict__ rscale,
                                                          const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                          int M, int N, int K, int TC, int rows_per_wg) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [TC][K]
  const int LDX = K;
  const int m0 = blockIdx.y * TC;
  const int tc = min(TC, M - m0);   // tokens of this chunk
  {
    // X[m0 .. m0 + tc) is one contiguous block: copied straight into LDS,
    // 1 KiB per wave instruction, the tail (a multiple of 64 bytes) by plain loads
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint16_t* src = X + (int64_t)m0 * K;
    const int nbytes = tc * K * 2, nfull = nbytes >> 10;
    for (int i = wave; i < nfull; i += kResThreads / 64)
      __builtin_amdgcn_global_load_lds(src + 512 * i + 8 * lane,
                                       (__attribute__((address_space(3))) void*)(xs + 512 * i), 16, 0, 0);
    const int tail = (nbytes - (nfull << 10)) >> 4;   // 16-byte granules
    if ((int)threadIdx.x < tail)
      reinterpret_cast<uint4*>(xs + 512 * nfull)[threadIdx.x] =
          reinterpret_cast<const uint4*>(src + 512 * nfull)[threadIdx.x];
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rend = min(N, (blockIdx.x + 1) * rows_per_wg);
  int row = blockIdx.x * rows_per_wg + wave;
  // current row: bounds, first 64 entries, Y of lane t's token
  int e0 = 0, e1 = 0, c;
  float q, y = 0.f;
  if (row < rend) {
    e0 = row_ptr[row];
    e1 = row_ptr[row + 1];
    if (lane < tc) y = h_to_f(Y[(int64_t)(m0 + lane) * N + row]);
  }
  load_entry(col, rcodes, e0 + lane, e1, c, q);
  for (; row < rend; row += kResThreads / 64) {
    const int nrow = row + kResThreads / 64;
    int ne0 = 0, ne1 = 0, nc;
    float nq, ny = 0.f;
    if (nrow < rend) {
      ne0 = row_ptr[nrow];
      ne1 = row_ptr[nrow + 1];
      if (lane < tc) ny = h_to_f(Y[(int64_t)(m0 + lane) * N + nrow]);
    }
    load_entry(col, rcodes, ne0 + lane, ne1, nc, nq);
    if (e1 > e0) {   // wave-uniform
      float mine = 0.f;
      if (e1 - e0 <= 64) {   // the common case: the row's entries are all in the lanes
        int t = 0;
        for (; t + 4 <= tc; t += 4) {   // four independent gathers and sums in flight
          float v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = q * h_to_f(xs[(t + u) * LDX + c]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float sum = wave_sum(v[u]);
            if (lane == t + u) mine = sum;
          }
        }
        for (; t < tc; ++t) {
          const float sum = wave_sum(q * h_to_f(xs[t * LDX + c]));
          if (lane == t) mine = sum;
        }
      } else {
        for (int t = 0; t < tc; ++t) {
          float v = q * h_to_f(xs[t * LDX + c]);
          for (int base = e0 + 64; base < e1; base += 64) {   // rows longer than 64 entries
            int c2;
            float q2;
            load_entry(col, rcodes, base + lane, e1, c2, q2);
            v += q2 * h_to_f(xs[t * LDX + c2]);
          }
          const float sum = wave_sum(v);
          if (lane == t) mine = sum;
        }
      }
      if (lane < tc) Y[(int64_t)(m0 + lane) * N + row] = f32_to_h(y + rscale[row] * mine);
    }
    e0 = ne0;
    e1 = ne1;
    c = nc;
    q = nq;
    y = ny;
  }
}

}  // namespace

hipError_t launch_residual(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t s) {
  if (p->nnz == 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_residual),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kResLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int K = (int)p->K, N = (int)p->N;
  // tokens per chunk: as many as M needs, at most 64 (one per lane) and as
  // many X rows as the LDS holds
  const int TC = (int)std::min<int64_t>({M, 64, kResLdsBytes / ((int64_t)K * 2)});   // K <= 65536: >= 1
  const int chunks = (int)((M + TC - 1) / TC);
  // about 256 workgroups of rows per token chunk, whole waves of rows each
  const int rows_per_wg = std::max(8, (int)((N + 255) / 256));
  const int groups = (N + rows_per_wg - 1) / rows_per_wg;
  const size_t lds = (size_t)TC * K * 2;
  k_residual<<<dim3((unsigned)groups, (unsigned)chunks), dim3(kResThreads), lds, s>>>(
      p->row_ptr, p->col, p->rcodes, p->rscale, X, Y, (int)M, N, K, TC, rows_per_wg);
  return hipGetLastError();
}

}  // namespace mq
