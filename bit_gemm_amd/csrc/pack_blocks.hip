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
//   4. k_block_codes: the selected blocks' scales and codes in canonical form
//      and their nonzero counts per row and per tile; k_block_pad rounds each
//      row block's stream segment up to whole 32-entry chunks;
//   5. k_block_emit: the residual stream the fused kernels read (entries with
//      fp16(sr qr), and the patched weights fp16(s q + fp16(sr qr))), in the
//      same (row block, tile, row, column) order as element-wise packing, so
//      the prefill and general decode kernels run these handles unchanged;
//      the blocks are also kept as 4-bit code tiles (with k_block_rtptr's
//      per-row-block ranges and k_block_slots' per-tile slots), which the
//      K = 4096 decode kernels multiply on the MFMA path like the base tiles
//      and the prefill GEMM widens into the weight tile it stages.
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
                                                       float* __restrict__ bscale, uint8_t* __restrict__ bcodes,
                                                       uint8_t* __restrict__ rt_tiles,
                                                       uint32_t* __restrict__ row_cnt,
                                                       uint32_t* __restrict__ tile_cnt,
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
  uint8_t* dst = bcodes + ((int64_t)n * kRowsPerBlock + r) * (kTileCols / 2) + 16 * kq;
#pragma unroll
  for (int t = 0; t < 16; ++t) dst[t] = (uint8_t)(u[r][32 * kq + 2 * t] | (u[r][32 * kq + 2 * t + 1] << 4));
  // the same codes in the code-tile layout (as the base tiles): lane r + 16 g,
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
  uint32_t ex, tot;
  row_lanes(nz, lane, &ex, &tot);
  if (kq == 0) row_cnt[(int64_t)n * kRowsPerBlock + r] = tot;
  uint32_t v = (kq == 0) ? tot : 0u;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o);
  if (lane == 0) {
    tile_cnt[b] = v;
    atomicAdd(nnz, (unsigned long long)v);
  }
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

// A row block's stream segment ends on a whole 32-entry chunk (zero entries).
__global__ __launch_bounds__(256) void k_block_pad(uint32_t* __restrict__ tile_cnt, int64_t Nb, int Kt) {
  const int64_t rb = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (rb >= Nb) return;
  uint32_t total = 0;
  for (int kt = 0; kt < Kt; ++kt) total += tile_cnt[rb * Kt + kt];
  if (total % kChunk) tile_cnt[rb * Kt + Kt - 1] += kChunk - total % kChunk;
}

// -------------------------------------------------------------- 5. emit
__global__ __launch_bounds__(kWave) void k_block_emit(const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ scales, int N, int K, int G,
                                                      int Kt, int64_t sstride, const int32_t* __restrict__ blk,
                                                      const uint32_t* __restrict__ row_cnt,
                                                      const uint32_t* __restrict__ tile_ptr,
                                                      const uint8_t* __restrict__ tiles,
                                                      uint32_t* __restrict__ entries, int64_t stream_cap,
                                                      SelState* flags) {
  const int n = blockIdx.x, b = blk[n], rb = b / Kt, kt = b - (b / Kt) * Kt;
  const int lane = threadIdx.x, r = lane & 15, kq = lane >> 4;
  BlockLane L;
  block_lane(W, scales, N, K, G, sstride, rb, kt, lane, L);
  int qr[32];
  uint32_t nz = 0;
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    qr[c] = L.t.valid ? quant7_scaled(L.e[c], L.sm, L.sQ) : 0;
    nz += (qr[c] != 0) ? 1u : 0u;
  }
  // entries of rows r' < r of the tile come first
  const uint32_t rc = row_cnt[(int64_t)n * kRowsPerBlock + r];
  uint32_t incl = rc;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const uint32_t x = (uint32_t)__shfl_up((int)incl, o, 16);
    if (r >= o) incl += x;
  }
  uint32_t ex, tot;
  row_lanes(nz, lane, &ex, &tot);
  if (!L.t.valid || nz == 0) return;
  uint32_t ps = tile_ptr[b] + (incl - rc) + ex;
  for (int c = 0; c < 32; ++c) {
    if (qr[c] == 0) continue;
    if ((int64_t)ps >= stream_cap) {   // counts disagree: never write out of bounds
      atomicOr(&flags->flags, kFlagCountMismatch);
      return;
    }
    const int j = L.t.c0 + c;
    // residual value sr qr = sm qr 2^(sQ - 24), rounded to fp16 for the kernels
    const _Float16 dh = (_Float16)ldexpf((float)((int64_t)L.sm * qr[c]), L.sQ - 24);
    entries[ps] = ((uint32_t)__builtin_bit_cast(uint16_t, dh) << 16) | ((uint32_t)r << 12) |
                  ((uint32_t)j & (kColWindow - 1));
    ++ps;
  }
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
  Temp t_state, t_keys, t_rc, t_tc, t_nnz;
  MQ_TRY(hipMalloc(&t_state.p, sizeof(SelState)));
  SelState* st = static_cast<SelState*>(t_state.p);
  MQ_TRY(hipMemsetAsync(st, 0, sizeof(SelState), stream));
  MQ_TRY(hipMemsetAsync(p->scales, 0, (size_t)Nb * kRowsPerBlock * p->sstride * sizeof(uint16_t), stream));
  MQ_TRY(hipMemsetAsync(p->tile_ptr, 0, (size_t)(ntiles + 1) * sizeof(uint32_t), stream));
  MQ_TRY(hipMemsetAsync(p->entries, 0, (size_t)(p->stream_cap + kEntryPad) * sizeof(uint32_t), stream));
  MQ_TRY(launch_pack_base(W, p, st, stream));
  // the all-zero block slot nblk: block 0's column tile, scales 0, codes 8 (q = 0)
  MQ_TRY(hipMemsetAsync(p->blk + nsel, 0, sizeof(int32_t), stream));
  MQ_TRY(hipMemsetAsync(p->bscale + nsel * kRowsPerBlock, 0, kRowsPerBlock * sizeof(float), stream));
  MQ_TRY(hipMemsetAsync(p->rt_tiles + nsel * kTileBytes, 0x88, kTileBytes, stream));
  MQ_TRY(hipMemsetAsync(p->rt_ptr, 0, (size_t)(Nb + 1) * sizeof(uint32_t), stream));
  k_block_slots<<<dim3((unsigned)((ntiles + 255) / 256)), dim3(256), 0, stream>>>(p->blk, nsel, ntiles, p->rt_slot);
  MQ_TRY(hipGetLastError());

  MQ_TRY(hipMalloc(&t_keys.p, (size_t)ntiles * sizeof(uint64_t)));
  MQ_TRY(hipMalloc(&t_tc.p, (size_t)ntiles * sizeof(uint32_t)));
  MQ_TRY(hipMalloc(&t_nnz.p, sizeof(unsigned long long)));
  MQ_TRY(hipMemsetAsync(t_tc.p, 0, (size_t)ntiles * sizeof(uint32_t), stream));
  MQ_TRY(hipMemsetAsync(t_nnz.p, 0, sizeof(unsigned long long), stream));
  uint64_t* keys = static_cast<uint64_t*>(t_keys.p);
  uint32_t* tcnt = static_cast<uint32_t*>(t_tc.p);
  k_block_scores<<<dim3((unsigned)ntiles), dim3(kWave), 0, stream>>>(W, p->scales, h, N, K, G, Kt, p->sstride,
                                                                     keys, st);
  MQ_TRY(hipGetLastError());
  if (nsel > 0) {
    MQ_TRY(hipMalloc(&t_rc.p, (size_t)nsel * kRowsPerBlock * sizeof(uint32_t)));
    uint32_t* rcnt = static_cast<uint32_t*>(t_rc.p);
    k_block_select<<<dim3(1), dim3(1024), 0, stream>>>(keys, ntiles, nsel, p->blk);
    MQ_TRY(hipGetLastError());
    k_block_codes<<<dim3((unsigned)nsel), dim3(kWave), 0, stream>>>(
        W, p->scales, N, K, G, Kt, p->sstride, p->blk, p->bscale, p->bcodes, p->rt_tiles, rcnt, tcnt,
        static_cast<unsigned long long*>(t_nnz.p));
    MQ_TRY(hipGetLastError());
    k_block_rtptr<<<dim3((unsigned)((Nb + 1 + 255) / 256)), dim3(256), 0, stream>>>(p->blk, nsel, Nb, Kt, p->rt_ptr);
    MQ_TRY(hipGetLastError());
    k_block_slots_set<<<dim3((unsigned)((nsel + 255) / 256)), dim3(256), 0, stream>>>(p->blk, nsel, p->rt_slot);
    MQ_TRY(hipGetLastError());
    k_block_pad<<<dim3((unsigned)((Nb + 255) / 256)), dim3(256), 0, stream>>>(tcnt, Nb, Kt);
    MQ_TRY(hipGetLastError());
    MQ_TRY(launch_scan_tiles(tcnt, ntiles, p->tile_ptr, st, stream));
    k_block_emit<<<dim3((unsigned)nsel), dim3(kWave), 0, stream>>>(W, p->scales, N, K, G, Kt, p->sstride, p->blk,
                                                                   rcnt, p->tile_ptr, p->tiles, p->entries,
                                                                   p->stream_cap, st);
    MQ_TRY(hipGetLastError());
  }
  SelState fin;
  uint32_t nstream = 0;
  unsigned long long nnz = 0;
  MQ_TRY(hipMemcpyAsync(&fin, st, sizeof(fin), hipMemcpyDeviceToHost, stream));
  MQ_TRY(hipMemcpyAsync(&nstream, p->tile_ptr + ntiles, sizeof(nstream), hipMemcpyDeviceToHost, stream));
  MQ_TRY(hipMemcpyAsync(&nnz, t_nnz.p, sizeof(nnz), hipMemcpyDeviceToHost, stream));
  MQ_TRY(hipStreamSynchronize(stream));
  *flags_out = fin.flags;
  p->nstream = nstream;
  p->nnz = (int64_t)nnz;
  if ((int64_t)nstream > p->stream_cap) *flags_out |= kFlagCountMismatch;
  return hipSuccess;
}

}  // namespace mq
