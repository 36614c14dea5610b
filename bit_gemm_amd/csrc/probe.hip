// Streaming-read probe: reads a device buffer once with 16-byte loads and
// folds it into one word per workgroup. It computes nothing of the layer; it
// gives the HBM read rate that a kernel streaming a buffer of a decode
// layer's size can reach on this chip, the practical ceiling the decode
// kernels' GB/s are set against.
#include "mq_internal.h"

namespace mq {
namespace {

// Workgroup b reads U = ceil(chunks / (workgroups * 256)) runs of 256
// consecutive 16-byte chunks from chunk b * 256 U on: thread t reads chunks
// b * 256 U + 256 u + t, u < U <= 16 (none past the end), every load issued
// before any is used, as a decode workgroup streams its code tiles. The XOR
// of everything it read goes to sink[b], so no load is dead.
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ src, int64_t nchunks, int U,
                                                     uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
  uint4 v[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t i = base + 256 * u;
    v[u] = (u < U && i < nchunks) ? src[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int t = 0; t < 256; ++t) s ^= red[t];
    sink[blockIdx.x] = s;
  }
}

}  // namespace

hipError_t stream_read(const void* src, int64_t bytes, int workgroups, uint32_t* sink, hipStream_t s) {
  const int64_t nchunks = bytes / 16;
  const int64_t U = (nchunks + (int64_t)workgroups * 256 - 1) / ((int64_t)workgroups * 256);
  if (U > 16) return hipErrorInvalidValue;   // rejected by the caller first
  k_stream_read<<<dim3((unsigned)workgroups), dim3(256), 0, s>>>(static_cast<const uint4*>(src), nchunks, (int)U,
                                                                 sink);
  return hipGetLastError();
}

}  // namespace mq
