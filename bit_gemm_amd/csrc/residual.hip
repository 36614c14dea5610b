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
// A workgroup (8 waves) owns a range of rows and a chunk of TC tokens: it
// copies X[m0 .. m0 + TC) into LDS once (row stride K + 2 halves, so the TC
// lanes that read one column of TC token rows hit different banks), then
// each wave takes one row at a time. The 64 lanes are TC tokens x (64 / TC)
// entry slots: slot s walks the row's entries s, s + 64/TC, ... and
// accumulates qr * x in fp32, the slots are summed with lane shuffles, and
// the slot-0 lanes add sr * sum to Y. Rows without entries are not touched.
#include <algorithm>

#include "kernel_common.h"
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int kResThreads = 512;
constexpr int kResLdsBytes = 160 * 1024;   // the whole LDS of a CU

__global__ __launch_bounds__(kResThreads) void k_residual(const int32_t* __restrict__ row_ptr,
                                                          const uint16_t* __restrict__ col,
                                                          const uint8_t* __restrict__ rcodes,
                                                          const float* __restrict__ rscale,
                                                          const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                                                          int M, int N, int K, int TC, int lg_tc, int rows_per_wg) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [TC][K + 2]
  const int LDX = K + 2;
  const int m0 = blockIdx.y * TC;
  const int tc = min(TC, M - m0);   // tokens of this chunk
  // stage X[m0 .. m0 + tc) (2-byte granules: the padded row stride is not 16-byte aligned)
  for (int idx = threadIdx.x; idx < tc * (K / 2); idx += kResThreads) {
    const int t = idx / (K / 2), c = 2 * (idx - t * (K / 2));
    const uint32_t v = *reinterpret_cast<const uint32_t*>(X + (int64_t)(m0 + t) * K + c);
    xs[t * LDX + c] = (uint16_t)v;
    xs[t * LDX + c + 1] = (uint16_t)(v >> 16);
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = lane & (TC - 1), slot = lane >> lg_tc, nslot = 64 >> lg_tc;
  const int row_end = min(N, (blockIdx.x + 1) * rows_per_wg);
  for (int row = blockIdx.x * rows_per_wg + wave; row < row_end; row += kResThreads / 64) {
    const int e0 = row_ptr[row], e1 = row_ptr[row + 1];
    if (e0 == e1) continue;   // wave-uniform
    float acc = 0.f;
    if (t < tc) {
      for (int e = e0 + slot; e < e1; e += nslot) {
        const int q = (int)((rcodes[e >> 1] >> (4 * (e & 1))) & 0xFu) - 8;
        acc += (float)q * h_to_f(xs[t * LDX + col[e]]);
      }
    }
    for (int o = TC; o < 64; o <<= 1) acc += __shfl_xor(acc, o);   // sum over the entry slots
    if (slot == 0 && t < tc) {
      uint16_t* y = Y + (int64_t)(m0 + t) * N + row;
      *y = f32_to_h(h_to_f(*y) + rscale[row] * acc);
    }
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
  // tokens per chunk: the largest power of two <= 64 whose X rows fit the LDS budget
  int lg = 6;
  while (lg > 0 && (int64_t)(1 << lg) * (K + 2) * 2 > kResLdsBytes) --lg;
  if ((int64_t)(K + 2) * 2 > kResLdsBytes) return hipErrorInvalidValue;   // one token row must fit
  const int TC = 1 << lg;
  const int chunks = (int)((M + TC - 1) / TC);
  // about 256 workgroups of rows per token chunk, whole waves of rows each
  const int rows_per_wg = std::max(8, (int)((N + 255) / 256));
  const int groups = (N + rows_per_wg - 1) / rows_per_wg;
  const size_t lds = (size_t)std::min<int64_t>(TC, M) * (K + 2) * 2;
  k_residual<<<dim3((unsigned)groups, (unsigned)chunks), dim3(kResThreads), lds, s>>>(
      p->row_ptr, p->col, p->rcodes, p->rscale, X, Y, (int)M, N, K, TC, lg, rows_per_wg);
  return hipGetLastError();
}

}  // namespace mq
