// Block-wise residual packing with a Hessian-guided score, on the GPU.
//
// MosaicQuant explainer, Methodology section 2 (Block-Wise Residual
// Allocation): the residual budget goes to blocks, chosen by a Delta-score
// that weights the residual error with the diagonal Hessian estimate of the
// input channels (the drop of the estimated output distortion when the block
// gets its residual); the top-K blocks receive a 4-bit residual.
//
// A block is one 16 x 128 code tile (row block rb, column tile kt). Steps:
//   1. the base codes and scales, as for element-wise packing;
//   2. k_block_scores: per block, the exact base errors e, per block row the
//      residual scale sr = fp32(max |e| / 7) and codes qr = clamp(rne(e / sr)),
//      and Delta = sum over rows, then columns, of h_j * (r * (2 e - r)),
//      r = sr * qr, each operation one float64 rounding (no contraction), the
//      sum taken left to right: the order is part of the definition, so the
//      score bits, and the selection, are reproducible;
//   3. k_block_select (one workgroup): radix select of the K-th largest score
//      (8 passes of 8 bits over the double's bit pattern), then the chosen
//      block indices in ascending order (ties at the threshold by index);
//   4. k_block_codes: the selected blocks' residual scales and codes, as
//      4-bit code tiles in the base tile layout (with k_block_rtptr's
//      per-row-block ranges and k_block_slots' per-tile slots): the decode,
//      mid-size and prefill kernels widen them like the base tiles (the
//      canonical codes are derived from these tiles on export).
#include "mq_internal.h"
#include "pack_common.h"
#include "quant_exact.h"

namespace mq {
namespace {

using namespace pack_detail;

// One lane's 32 entries of block (rb, kt): exact base errors (units of
// 2^-24) and the residual scale of the lane's block row (fp32 bits, and as
// sm * 2^sQ units).
struct BlockLane {
  LaneTile t;
  int64_t e[32];
  uint64_t sm;
  int sQ;
  uint32_t srbits;
};

__device__ __forceinline__ void block_lane(const uint16_t* __restrict__ W, const uint16_t* __restrict__ scales,
                                           int N, int K, int G, int64_t sstride, int rb, int kt, int lane,
                                           BlockLane& L) {
  L.t = lane_tile(rb, kt, lane, N, K);
  uint64_t amax = 0;
  if (L.t.valid) {
    uint32_t w[16];
    uint64_t key[32];
    load32(W, K, L.t, w);
    keys_from_w(w, lane_scale_units(scales, sstride, G, L.t), key, L.e);
#pragma unroll
    for (int c = 0; c < 32; ++c) amax = max(amax, (uint64_t)(L.e[c] < 0 ? -L.e[c] : L.e[c]));
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) L.e[c] = 0;
  }
  // the block row's four lanes
  amax = max(amax, (uint64_t)__shfl_xor((unsigned long long)amax, 16));
  amax = max(amax, (uint64_t)__shfl_xor((unsigned long long)amax, 32));
  L.srbits = fp32_div7(amax, &L.sm, &L.sQ);
}

// ------------------------------------------------------------ 2. scores
__global__ __launch_bounds__(kWave) void k_block_scores(const uint16_t* __restrict__ W,
                                                        const uint16_t* __restrict__ scales,
                                                        const float* __restrict__ h, int N, int K, int G, int Kt,
                                                        int64_t sstride, uint64_t* __restrict__ keys,
                                                        SelState* st) {
#pragma clang fp contract(off)
  __shared__ double term[kRowsPerBlock][kTileCols];
  const int b = blockIdx.x, rb = b / Kt, kt = b - (b / Kt) * Kt;
  const int lane = threadIdx.x, r = lane & 15, kq = lane >> 4;
  BlockLane L;
  block_lane(W, scales, N, K, G, sstride, rb, kt, lane, L);
  const double sr = (double)__builtin_bit_cast(float, L.srbits);
  bool bad = false;
#pragma unroll 4
  for (int c = 0; c < 32; ++c) {
    double t = 0.0;
    if (L.t.valid) {
      const float hf = h[L.t.c0 + c];
      bad |= !(hf >= 0.0f && hf <= 3.4028234663852886e38f);   // negative, inf or NaN
      const double rr = sr * (double)quant7_scaled(L.e[c], L.sm, L.sQ);   // exact
      const double ed = (double)L.e[c] * 0x1p-24;                         // exact
      t = (double)hf * (rr * (2.0 * ed - rr));
    }
    term[r][32 * kq + c] = t;
  }
  if (bad) atomicOr(&st->flags, kFlagBadHessian);
  __syncthreads();
  if (lane == 0) {
    const int rows = min(kRowsPerBlock, N - rb * kRowsPerBlock), cols = min(kTileCols, K - kt * kTileCols);
    double acc = 0.0;
    for (int i = 0; i < rows; ++i)
      for (int j = 0; j < cols; ++j) acc += term[i][j];   // rows, then columns, left to right
    if (acc == 0.0) acc = 0.0;                           // one key for +0 and -0
    keys[b] = __builtin_bit_cast(uint64_t, acc);         // scores are >= 0: bit order == value order
  }
}

// ------------------------------------------------------------ 3. select
// One workgroup of 1024 threads. K-th largest key by 8 radix passes of 8
// bits, then one pass in index order that takes every key above it and the
// first `krem` keys equal to it, writing the chosen indices in ascending
// order.
__global__ __launch_bounds__(1024) void k_block_select(const uint64_t* __restrict__ keys, int64_t nblk, int64_t k,
                                                       int32_t* __restrict__ blk) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t wave_tot[16];
  __shared__ uint64_t sh_prefix, sh_krem, sh_tot;
  const int tid = threadIdx.x;
  uint64_t prefix = 0, mask = 0, krem = (uint64_t)k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < nblk; i += blockDim.x) {
      const uint64_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint64_t cum = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (cum + hist[d] >= krem) break;
        cum += hist[d];
      }
      sh_prefix = prefix | ((uint64_t)d << shift);
      sh_krem = krem - cum;
    }
    __syncthreads();
    prefix = sh_prefix;
    krem = sh_krem;
    mask |= 255ull << shift;
    __syncthreads();
  }
  const uint64_t T = prefix;
  uint64_t carry_tie = 0, carry_sel = 0;
  for (int64_t base = 0; base < nblk; base += blockDim.x) {
    const int64_t i = base + tid;
    const uint64_t key = (i < nblk) ? keys[i] : 0ull;
    const uint64_t eq = (i < nblk && key == T) ? 1u : 0u;
    const uint64_t tie_incl = block_scan_incl(eq, wave_tot);
    const uint64_t tie_rank = carry_tie + tie_incl - eq;
    if (tid == (int)blockDim.x - 1) sh_tot = tie_incl;
    __syncthreads();
    carry_tie += sh_tot;
    __syncthreads();
    const uint64_t sel = (i < nblk && (key > T || (eq && tie_rank < krem))) ? 1u : 0u;
    const uint64_t sel_incl = block_scan_incl(sel, wave_tot);
    if (sel) blk[carry_sel + sel_incl - 1] = (int32_t)i;
    if (tid == (int)blockDim.x - 1) sh_tot = sel_incl;
    __syncthreads();
    carry_sel += sh_tot;
    __syncthreads();
  }
}

// ------------------------------------------------------------- 4. codes
__global__ __launch_bounds__(kWave) void k_block_codes(const uint16_t* __restrict__ W,
                                                       const uint16_t* __restrict__ scales, int N, int K, int G,
                                                       int Kt, int64_t sstride, const int32_t* __restrict__ blk,
                                                       float* __restrict__ bscale, uint8_t* __restrict__ rt_tiles,
                                                       unsigned long long* __restrict__ nnz) {
  __shared__ uint8_t u[kRowsPerBlock][kTileCols];
  const int n = blockIdx.x, b = blk[n], rb = b / Kt, kt = b - (b / Kt) * Kt;
  const int lane = threadIdx.x, r = lane & 15, kq = lane >> 4;
  BlockLane L;
  block_lane(W, scales, N, K, G, sstride, rb, kt, lane, L);
  uint32_t nz = 0;
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const int qr = L.t.valid ? quant7_scaled(L.e[c], L.sm, L.sQ) : 0;
    u[r][32 * kq + c] = (uint8_t)(qr + 8);
    nz += (qr != 0) ? 1u : 0u;
  }
  if (kq == 0) bscale[(int64_t)n * kRowsPerBlock + r] = __builtin_bit_cast(float, L.srbits);
  __syncthreads();
  // the codes in the code-tile layout (as the base tiles): lane r + 16 g,
  // dword s4 holds columns 32 s4 + 8 g + c at nibble nib_pos(c)
  uint32_t d[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    uint32_t v = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) v |= (uint32_t)u[r][32 * s4 + 8 * kq + c] << (4 * nib_pos(c));
    d[s4] = v;
  }
  reinterpret_cast<uint4*>(rt_tiles)[(int64_t)n * kWave + lane] = make_uint4(d[0], d[1], d[2], d[3]);
  // the block's nonzero residual codes, counted into nnz
  uint32_t v = nz;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o);
  if (lane == 0) atomicAdd(nnz, (unsigned long long)v);
}

// rt_ptr[rb] = first selected block of row block rb (blk is ascending, so a
// row block's blocks are contiguous): a lower bound by binary search.
__global__ __launch_bounds__(256) void k_block_rtptr(const int32_t* __restrict__ blk, int64_t nsel, int64_t Nb,
                                                     int Kt, uint32_t* __restrict__ rt_ptr) {
  const int64_t rb = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (rb > Nb) return;
  const int64_t key = rb * Kt;
  int64_t lo = 0, hi = nsel;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if ((int64_t)blk[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  rt_ptr[rb] = (uint32_t)lo;
}

// rt_slot[b] = n for the n-th selected block b, the zero slot nsel elsewhere.
__global__ __launch_bounds__(256) void k_block_slots(const int32_t* __restrict__ blk, int64_t nsel, int64_t ntiles,
                                                     int32_t* __restrict__ rt_slot) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < ntiles) rt_slot[i] = (int32_t)nsel;
}

__global__ __launch_bounds__(256) void k_block_slots_set(const int32_t* __restrict__ blk, int64_t nsel,
                                                         int32_t* __restrict__ rt_slot) {
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n < nsel) rt_slot[blk[n]] = (int32_t)n;
}

struct Temp {
  void* p = nullptr;
  ~Temp() {
    if (p) (void)hipFree(p);
  }
};

}  // namespace

#define MQ_TRY(x)                        \
  do {                                   \
    hipError_t err_ = (x);               \
    if (err_ != hipSuccess) return err_; \
  } while (0)

hipError_t pack_blocks_on_device(const uint16_t* W, const float* h, mq_packed* p, hipStream_t stream,
                                 uint32_t* flags_out) {
  const int N = (int)p->N, K = (int)p->K, G = p->G, Kt = (int)p->Kt;
  const int64_t Nb = p->Nb, ntiles = Nb * Kt, nsel = p->nblk;
  Temp t_state, t_keys, t_nnz;
  MQ_TRY(hipMalloc(&t_state.p, sizeof(SelState)));
  SelState* st = static_cast<SelState*>(t_state.p);
  MQ_TRY(hipMemsetAsync(st, 0, sizeof(SelState), stream));
  MQ_TRY(hipMemsetAsync(p->scales, 0, (size_t)Nb * kRowsPerBlock * p->sstride * sizeof(uint16_t), stream));
  MQ_TRY(launch_pack_base(W, p, st, stream));
  // the all-zero block slot nblk: block 0's column tile, scales 0, codes 8 (q = 0)
  MQ_TRY(hipMemsetAsync(p->blk + nsel, 0, sizeof(int32_t), stream));
  MQ_TRY(hipMemsetAsync(p->bscale + nsel * kRowsPerBlock, 0, kRowsPerBlock * sizeof(float), stream));
  MQ_TRY(hipMemsetAsync(p->rt_tiles + nsel * kTileBytes, 0x88, kTileBytes, stream));
  MQ_TRY(hipMemsetAsync(p->rt_ptr, 0, (size_t)(Nb + 1) * sizeof(uint32_t), stream));
  k_block_slots<<<dim3((unsigned)((ntiles + 255) / 256)), dim3(256), 0, stream>>>(p->blk, nsel, ntiles, p->rt_slot);
  MQ_TRY(hipGetLastError());

  MQ_TRY(hipMalloc(&t_keys.p, (size_t)ntiles * sizeof(uint64_t)));
  MQ_TRY(hipMalloc(&t_nnz.p, sizeof(unsigned long long)));
  MQ_TRY(hipMemsetAsync(t_nnz.p, 0, sizeof(unsigned long long), stream));
  uint64_t* keys = static_cast<uint64_t*>(t_keys.p);
  k_block_scores<<<dim3((unsigned)ntiles), dim3(kWave), 0, stream>>>(W, p->scales, h, N, K, G, Kt, p->sstride,
                                                                     keys, st);
  MQ_TRY(hipGetLastError());
  if (nsel > 0) {
    k_block_select<<<dim3(1), dim3(1024), 0, stream>>>(keys, ntiles, nsel, p->blk);
    MQ_TRY(hipGetLastError());
    k_block_codes<<<dim3((unsigned)nsel), dim3(kWave), 0, stream>>>(
        W, p->scales, N, K, G, Kt, p->sstride, p->blk, p->bscale, p->rt_tiles,
        static_cast<unsigned long long*>(t_nnz.p));
    MQ_TRY(hipGetLastError());
    k_block_rtptr<<<dim3((unsigned)((Nb + 1 + 255) / 256)), dim3(256), 0, stream>>>(p->blk, nsel, Nb, Kt, p->rt_ptr);
    MQ_TRY(hipGetLastError());
    k_block_slots_set<<<dim3((unsigned)((nsel + 255) / 256)), dim3(256), 0, stream>>>(p->blk, nsel, p->rt_slot);
    MQ_TRY(hipGetLastError());
  }
  SelState fin;
  unsigned long long nnz = 0;
  MQ_TRY(hipMemcpyAsync(&fin, st, sizeof(fin), hipMemcpyDeviceToHost, stream));
  MQ_TRY(hipMemcpyAsync(&nnz, t_nnz.p, sizeof(nnz), hipMemcpyDeviceToHost, stream));
  MQ_TRY(hipStreamSynchronize(stream));
  *flags_out = fin.flags;
  p->nnz = (int64_t)nnz;
  return hipSuccess;
}

}  // namespace mq
