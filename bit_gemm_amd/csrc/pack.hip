// Packer: W (fp16) -> dense 4-bit base + sparse 4-bit residual, on the GPU.
//
// Steps (MosaicQuant explainer, Methodology section 1, Eq. (1) W ~ Q(W) + R;
// section 2, residual budget given to the top-K scoring units):
//   1. k_pack_base   per (row, group): fp16 scale of absmax/7, base codes,
//                    written straight into the kernels' tile layout;
//   2. k_hist + k_select_digit, 4 passes: exact radix select of the k-th
//                    largest |e| over the whole matrix (keys never stored, they
//                    are recomputed from W and the scales);
//   3. k_row_counts / k_scan_rows: per-row counts above / at the threshold,
//                    ties ranked by row-major index, CSR row pointer;
//   4. k_row_select: per-row residual scale fp32(max selected |e| / 7) and
//                    per-(row, tile) entry counts; k_scan_tiles: tile pointer;
//   5. k_row_emit:   CSR columns and residual codes, and the residual stream
//                    the fused kernels read (sorted by row block, tile, row, col).
// All arithmetic is exact integer arithmetic (quant_exact.h) and every
// reduction has a fixed order, so the result is bit-identical run to run.
#include "mq_internal.h"
#include "pack_common.h"
#include "quant_exact.h"

#include <algorithm>
#include <cmath>

namespace mq {
namespace {

using namespace pack_detail;



// ---------------------------------------------------------------- 1. base
// The wave computes the codes of one 16 x 128 tile (lane l: row l % 16,
// columns 32 (l / 16) .. +32), then rewrites them through LDS into the kernel
// layout, where lane l = r + 16 g holds in dword t the columns 32 t + 8 g + c,
// c = 0..7, at nibble (c / 2) + 4 (c % 2): a dword is then exactly the A
// operand of one 16x16x32 MFMA step over 32 consecutive columns.
__global__ __launch_bounds__(kWave) void k_pack_base(const uint16_t* __restrict__ W, int N, int K, int G,
                                                     int Kt, int64_t sstride, uint8_t* __restrict__ tiles,
                                                     uint16_t* __restrict__ scales, SelState* st) {
  __shared__ uint8_t ucode[kRowsPerBlock][kTileCols];
  const int tile = blockIdx.x;
  const int rb = tile / Kt, kt = tile - (tile / Kt) * Kt;
  const int lane = threadIdx.x;
  const LaneTile t = lane_tile(rb, kt, lane, N, K);
  const int r = lane & 15, kq = lane >> 4;
  uint32_t w[16];
  uint32_t amax = 0;
  bool finite = true;
  if (t.valid) {
    load32(W, K, t, w);
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const uint32_t h = half_at(w, c);
      finite &= fp16_is_finite(h);
      amax = max(amax, h & 0x7FFFu);   // magnitude order == bit order for finite fp16
    }
  }
  if (G >= 64) amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16));
  if (G >= 128) amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
  if (!finite) atomicOr(&st->flags, kFlagNonFinite);

  uint8_t* myrow = &ucode[r][32 * kq];
  if (t.valid && finite) {
    uint64_t S;
    const uint32_t sbits = fp16_div7((uint64_t)fp16_units(amax), &S);
    // 7 s must stay finite in fp16: the prefill kernel forms s*q in fp16
    if (7u * S > (2047ull << 29)) atomicOr(&st->flags, kFlagScaleOverflow);
#pragma unroll
    for (int c = 0; c < 32; ++c) myrow[c] = (uint8_t)(quant7(fp16_units(half_at(w, c)), S) + 8);
    if ((t.c0 % G) == 0) scales[(int64_t)t.row * sstride + t.c0 / G] = (uint16_t)sbits;
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) myrow[c] = 8u;   // padding: q = 0
  }
  __syncthreads();
  uint32_t d[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    uint32_t v = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) v |= (uint32_t)ucode[r][32 * s4 + 8 * kq + c] << (4 * nib_pos(c));
    d[s4] = v;
  }
  reinterpret_cast<uint4*>(tiles)[(int64_t)tile * kWave + lane] = make_uint4(d[0], d[1], d[2], d[3]);
}


// ------------------------------------------------------- 2. radix select
__global__ __launch_bounds__(256) void k_hist(const uint16_t* __restrict__ W, const uint16_t* __restrict__ scales,
                                              int N, int K, int G, int Kt, int64_t sstride, int ntiles, int pass,
                                              const SelState* __restrict__ st, uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[kDigitBins];
  for (int i = threadIdx.x; i < kDigitBins; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  const int shift = 51 - kDigitBits * pass;
  // bits above this digit are fixed by the earlier passes
  const uint64_t fixed = (pass == 0) ? 0ull : (~0ull << (shift + kDigitBits));
  const uint64_t want = st->prefix & fixed;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int waves = blockDim.x / kWave;
  for (int tile = blockIdx.x * waves + wave; tile < ntiles; tile += gridDim.x * waves) {
    const int rb = tile / Kt, kt = tile - (tile / Kt) * Kt;
    const LaneTile t = lane_tile(rb, kt, lane, N, K);
    if (!t.valid) continue;
    uint64_t key[32];
    int64_t e[32];
    lane_keys(W, scales, K, G, sstride, t, key, e);
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      if ((key[c] & fixed) == want) atomicAdd(&h[(key[c] >> shift) & (kDigitBins - 1)], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kDigitBins; i += blockDim.x)
    if (h[i]) atomicAdd(&hist[i], h[i]);
}


// One block of 1024 threads: find the digit of the krem-th largest key among
// keys that match the prefix, scanning bins from the largest digit down.
__global__ __launch_bounds__(1024) void k_select_digit(uint32_t* __restrict__ hist, SelState* st, int pass) {
  __shared__ uint64_t wave_tot[16];
  constexpr int per = kDigitBins / 1024;
  const int t = threadIdx.x;
  const uint64_t krem = st->krem;
  uint32_t local[per];
  uint64_t s = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    local[i] = hist[kDigitBins - 1 - (per * t + i)];
    s += local[i];
  }
  const uint64_t incl = block_scan_incl(s, wave_tot);
  const uint64_t excl = incl - s;
  if (excl < krem && krem <= incl) {
    uint64_t c = excl;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      if (c + local[i] >= krem) {
        const uint64_t digit = (uint64_t)(kDigitBins - 1 - (per * t + i));
        st->prefix |= digit << (51 - kDigitBits * pass);
        st->krem = krem - c;
        break;
      }
      c += local[i];
    }
  }
#pragma unroll
  for (int i = 0; i < per; ++i) hist[kDigitBins - 1 - (per * t + i)] = 0u;
}


// ----------------------------------------------- 3. per-row threshold counts
__global__ __launch_bounds__(kWave) void k_row_counts(const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ scales, int N, int K, int G,
                                                      int Kt, int64_t sstride, const SelState* __restrict__ st,
                                                      uint32_t* __restrict__ cnt_gt, uint32_t* __restrict__ cnt_eq) {
  const int rb = blockIdx.x, lane = threadIdx.x;
  const uint64_t T = st->prefix;
  uint32_t gt = 0, eq = 0;
  for (int kt = 0; kt < Kt; ++kt) {
    const LaneTile t = lane_tile(rb, kt, lane, N, K);
    if (!t.valid) continue;
    uint64_t key[32];
    int64_t e[32];
    lane_keys(W, scales, K, G, sstride, t, key, e);
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      gt += key[c] > T ? 1u : 0u;
      eq += key[c] == T ? 1u : 0u;
    }
  }
  uint32_t ex, tot_gt, tot_eq;
  row_lanes(gt, lane, &ex, &tot_gt);
  row_lanes(eq, lane, &ex, &tot_eq);
  const int row = rb * kRowsPerBlock + (lane & 15);
  if ((lane >> 4) == 0 && row < N) {
    cnt_gt[row] = tot_gt;
    cnt_eq[row] = tot_eq;
  }
}

// One block of 1024 threads: tie ranks per row (ties are taken in row-major
// index order) and the CSR row pointer of the selected entries.
__global__ __launch_bounds__(1024) void k_scan_rows(const uint32_t* __restrict__ cnt_gt,
                                                    const uint32_t* __restrict__ cnt_eq, int N,
                                                    SelState* st, uint32_t* __restrict__ eq_base,
                                                    int32_t* __restrict__ row_ptr, uint64_t k_total) {
  __shared__ uint64_t wave_tot[16];
  const uint64_t krem = st->krem;
  uint64_t carry_eq = 0, carry_sel = 0;
  for (int base = 0; base < N; base += blockDim.x) {
    const int i = base + threadIdx.x;
    const uint64_t ceq = (i < N) ? cnt_eq[i] : 0u;
    const uint64_t cgt = (i < N) ? cnt_gt[i] : 0u;
    const uint64_t eq_incl = block_scan_incl(ceq, wave_tot);
    const uint64_t eb = carry_eq + eq_incl - ceq;
    const uint64_t room = (krem > eb) ? krem - eb : 0ull;
    const uint64_t take = room < ceq ? room : ceq;
    const uint64_t sel = cgt + take;
    const uint64_t sel_incl = block_scan_incl(sel, wave_tot);
    if (i < N) {
      eq_base[i] = (uint32_t)eb;
      row_ptr[i] = (int32_t)(carry_sel + sel_incl - sel);
    }
    // totals of this chunk come from the last thread
    __shared__ uint64_t tot[2];
    if (threadIdx.x == blockDim.x - 1) {
      tot[0] = eq_incl;
      tot[1] = sel_incl;
    }
    __syncthreads();
    carry_eq += tot[0];
    carry_sel += tot[1];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    row_ptr[N] = (int32_t)carry_sel;
    if (carry_sel != k_total) atomicOr(&st->flags, kFlagCountMismatch);
  }
}

// Selection flags of one lane's 32 entries in column order.
// tie_rank0 = rank (row-major order over the whole matrix) of this lane's
// first entry whose key equals T.
__device__ __forceinline__ uint32_t lane_select(const uint64_t (&key)[32], uint64_t T, uint64_t tie_rank0,
                                                uint64_t krem) {
  uint32_t sel = 0;
  uint64_t tr = tie_rank0;
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const bool eq = key[c] == T;
    const bool s = (key[c] > T) || (eq && tr < krem);
    tr += eq ? 1u : 0u;
    sel |= (s ? 1u : 0u) << c;
  }
  return sel;
}

__device__ __forceinline__ uint32_t lane_eq_count(const uint64_t (&key)[32], uint64_t T) {
  uint32_t n = 0;
#pragma unroll
  for (int c = 0; c < 32; ++c) n += (key[c] == T) ? 1u : 0u;
  return n;
}

// ---------------------------------- 4. residual scales and per-tile counts
__global__ __launch_bounds__(kWave) void k_row_select(const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ scales, int N, int K, int G,
                                                      int Kt, int64_t sstride, const SelState* __restrict__ st,
                                                      const uint32_t* __restrict__ eq_base,
                                                      float* __restrict__ rscale, uint32_t* __restrict__ cnt_rt,
                                                      uint32_t* __restrict__ tile_cnt) {
  const int rb = blockIdx.x, lane = threadIdx.x;
  const uint64_t T = st->prefix, krem = st->krem;
  const int row = rb * kRowsPerBlock + (lane & 15);
  const uint64_t ebase = (row < N) ? eq_base[row] : 0u;
  uint64_t run_tie = 0;      // ties of this row in earlier tiles
  uint64_t maxkey = 0;
  uint32_t rb_total = 0;     // stream entries of the row block (lane 0)
  for (int kt = 0; kt < Kt; ++kt) {
    const LaneTile t = lane_tile(rb, kt, lane, N, K);
    uint64_t key[32];
    int64_t e[32];
    uint32_t sel = 0, neq = 0;
    if (t.valid) {
      lane_keys(W, scales, K, G, sstride, t, key, e);
      neq = lane_eq_count(key, T);
    }
    uint32_t tie_ex, tie_tot;
    row_lanes(neq, lane, &tie_ex, &tie_tot);
    if (t.valid) {
      sel = lane_select(key, T, ebase + run_tie + tie_ex, krem);
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if ((sel >> c) & 1u) maxkey = max(maxkey, key[c]);
    }
    run_tie += tie_tot;
    uint32_t sel_ex, sel_tot;
    row_lanes((uint32_t)__popc(sel), lane, &sel_ex, &sel_tot);
    if ((lane >> 4) == 0 && row < N) cnt_rt[(int64_t)row * Kt + kt] = sel_tot;
    // tile total over the 16 rows
    uint32_t v = ((lane >> 4) == 0) ? sel_tot : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o);
    if (lane == 0) tile_cnt[(int64_t)rb * Kt + kt] = v;
    rb_total += v;
  }
  // pad the row block's stream segment to whole 32-entry chunks (zero entries)
  if (lane == 0 && (rb_total % kChunk) != 0)
    tile_cnt[(int64_t)rb * Kt + Kt - 1] += kChunk - rb_total % kChunk;
  // max over the row's four lanes
  maxkey = max(maxkey, (uint64_t)__shfl_xor((unsigned long long)maxkey, 16));
  maxkey = max(maxkey, (uint64_t)__shfl_xor((unsigned long long)maxkey, 32));
  if ((lane >> 4) == 0 && row < N) {
    const uint64_t mx = (uint64_t)__builtin_bit_cast(double, maxkey);   // keys are exact doubles
    uint64_t m;
    int Q;
    const uint32_t bits = fp32_div7(mx, &m, &Q);
    rscale[row] = __builtin_bit_cast(float, bits);
  }
}

// One block of 1024 threads: exclusive scan of the per-tile entry counts,
// their maximum into st->max_seg, the longest row block (Kt tiles) into
// st->max_rb, and the row blocks of more than kDenseRbChunks chunks: their
// count into st->ndense and (dense_rb not null) the first kDenseListMax of
// them, ascending, into dense_rb[0 .. 64), with their first stream entry
// and chunk count in dense_rb[64 ..) and dense_rb[128 ..). A decode launch
// that takes these row blocks first, knowing their streams without a load,
// starts its slowest workgroups in its first round.
__global__ __launch_bounds__(1024) void k_scan_tiles(const uint32_t* __restrict__ tile_cnt, int64_t ntiles, int64_t Kt,
                                                     uint32_t* __restrict__ tile_ptr,
                                                     uint32_t* __restrict__ dense_rb, SelState* st) {
  __shared__ uint64_t wave_tot[16];
  __shared__ uint64_t tot;
  __shared__ uint32_t seg_max;
  if (threadIdx.x == 0) seg_max = 0u;
  uint64_t carry = 0;
  uint32_t mx = 0u;
  for (int64_t base = 0; base < ntiles; base += blockDim.x) {
    const int64_t i = base + threadIdx.x;
    const uint64_t v = (i < ntiles) ? tile_cnt[i] : 0u;
    mx = max(mx, (uint32_t)v);
    const uint64_t incl = block_scan_incl(v, wave_tot);
    if (i < ntiles) tile_ptr[i] = (uint32_t)(carry + incl - v);
    if (threadIdx.x == blockDim.x - 1) tot = incl;
    __syncthreads();
    carry += tot;
    __syncthreads();
  }
  atomicMax(&seg_max, mx);
  if (threadIdx.x == 0) tile_ptr[ntiles] = (uint32_t)carry;
  __syncthreads();   // the block's tile_ptr writes are visible to all its threads
  __shared__ uint32_t rb_max;
  if (threadIdx.x == 0) rb_max = 0u;
  __syncthreads();
  __shared__ uint32_t ndense;
  if (threadIdx.x == 0) ndense = 0u;
  __syncthreads();
  const int64_t Nb = ntiles / Kt;
  auto dense = [&](int64_t rb) { return tile_ptr[(rb + 1) * Kt] - tile_ptr[rb * Kt] > (uint32_t)(kChunk * kDenseRbChunks); };
  uint32_t rmx = 0u, nd = 0u;
  for (int64_t rb = threadIdx.x; rb < Nb; rb += blockDim.x) {
    rmx = max(rmx, tile_ptr[(rb + 1) * Kt] - tile_ptr[rb * Kt]);
    nd += dense(rb) ? 1u : 0u;
  }
  atomicMax(&rb_max, rmx);
  atomicAdd(&ndense, nd);
  __syncthreads();
  if (dense_rb) {
    uint64_t before = 0;   // dense row blocks ahead of this tile of row blocks
    for (int64_t base = 0; base < Nb && before < (uint64_t)kDenseListMax; base += blockDim.x) {
      const int64_t rb = base + threadIdx.x;
      const uint64_t f = (rb < Nb && dense(rb)) ? 1u : 0u;
      const uint64_t incl = block_scan_incl(f, wave_tot);
      const uint64_t d = before + incl - f;   // dense row blocks before rb
      if (f && d < (uint64_t)kDenseListMax) {
        const uint32_t e0 = tile_ptr[rb * Kt];
        dense_rb[d] = (uint32_t)rb;
        dense_rb[kDenseListMax + d] = e0;
        dense_rb[2 * kDenseListMax + d] = (tile_ptr[(rb + 1) * Kt] - e0) / (uint32_t)kChunk;
      }
      if (threadIdx.x == blockDim.x - 1) tot = incl;
      __syncthreads();
      before += tot;
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    st->max_seg = seg_max;
    st->max_rb = rb_max;
    st->ndense = ndense;
  }
}

// ------------------------------------------------- 5. emit CSR and stream
__global__ __launch_bounds__(kWave) void k_row_emit(const uint16_t* __restrict__ W,
                                                    const uint16_t* __restrict__ scales, int N, int K, int G,
                                                    int Kt, int64_t sstride, const SelState* st,
                                                    const uint32_t* __restrict__ eq_base,
                                                    const int32_t* __restrict__ row_ptr,
                                                    const float* __restrict__ rscale,
                                                    const uint32_t* __restrict__ cnt_rt,
                                                    const uint32_t* __restrict__ tile_ptr,
                                                    const uint8_t* __restrict__ tiles,
                                                    uint16_t* __restrict__ col, uint32_t* __restrict__ rcodes32,
                                                    uint32_t* __restrict__ entries, uint32_t* __restrict__ wpatch,
                                                    int64_t nnz,
                                                    int64_t stream_cap, SelState* flags) {
  const int rb = blockIdx.x, lane = threadIdx.x;
  const int r = lane & 15;
  const uint64_t T = st->prefix, krem = st->krem;
  const int row = rb * kRowsPerBlock + r;
  const bool row_ok = row < N;
  const uint64_t ebase = row_ok ? eq_base[row] : 0u;
  uint64_t sm = 0;
  int sQ = 0;
  if (row_ok) fp32_units(__builtin_bit_cast(uint32_t, rscale[row]), &sm, &sQ);
  int64_t csr = row_ok ? row_ptr[row] : 0;
  uint64_t run_tie = 0;
  for (int kt = 0; kt < Kt; ++kt) {
    const LaneTile t = lane_tile(rb, kt, lane, N, K);
    uint32_t w[16];
    uint64_t key[32];
    int64_t e[32];
    uint64_t S = 0;
    uint32_t sel = 0, neq = 0;
    if (t.valid) {
      load32(W, K, t, w);
      S = lane_scale_units(scales, sstride, G, t);
      keys_from_w(w, S, key, e);
      neq = lane_eq_count(key, T);
    }
    uint32_t tie_ex, tie_tot;
    row_lanes(neq, lane, &tie_ex, &tie_tot);
    if (t.valid) sel = lane_select(key, T, ebase + run_tie + tie_ex, krem);
    run_tie += tie_tot;
    uint32_t sel_ex, sel_tot;
    row_lanes((uint32_t)__popc(sel), lane, &sel_ex, &sel_tot);
    // stream offset of this row inside the tile: entries of rows r' < r come first
    const uint32_t rc = row_ok ? cnt_rt[(int64_t)row * Kt + kt] : 0u;   // same on the row's 4 lanes
    uint32_t incl = rc;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const uint32_t u = (uint32_t)__shfl_up((int)incl, o, 16);
      if (r >= o) incl += u;
    }
    const uint32_t row_off = incl - rc;
    if (sel) {
      int64_t pc = csr + sel_ex;
      uint32_t ps = tile_ptr[(int64_t)rb * Kt + kt] + row_off + sel_ex;
      // the lane's base scale and the tile's codes, for the patched weight
      const float sbase = (float)__builtin_bit_cast(_Float16, scales[(int64_t)row * sstride + t.c0 / G]);
      const uint32_t* tw = reinterpret_cast<const uint32_t*>(tiles) + ((int64_t)rb * Kt + kt) * (kWave * 4);
      for (int c = 0; c < 32; ++c) {
        if (!((sel >> c) & 1u)) continue;
        const int j = t.c0 + c;
        if (pc >= nnz || (int64_t)ps >= stream_cap) {   // counts disagree: never write out of bounds
          atomicOr(&flags->flags, kFlagCountMismatch);
          break;
        }
        const int qr = quant7_scaled(e[c], sm, sQ);
        col[pc] = (uint16_t)j;
        atomicOr(&rcodes32[pc >> 3], (uint32_t)(qr + 8) << (4 * (pc & 7)));
        // Correction the fused kernels add to the base weight s q: the
        // residual value sr qr = m qr 2^(Q-24) in fp16 (|m qr| < 2^27, so the
        // float is within 2^-24 relative; the fp16 rounding dominates).
        const float dres = ldexpf((float)((int64_t)sm * qr), sQ - 24);
        const _Float16 dh = (_Float16)dres;
        entries[ps] = ((uint32_t)__builtin_bit_cast(uint16_t, dh) << 16) | ((uint32_t)r << 12) |
                      ((uint32_t)j & (kColWindow - 1));
        // Patch for the GEMM kernels, which widen the base weight to
        // fp16(s q) (the exact product, rounded once, as their packed
        // multiply forms it): the patched weight fp16(s q + fp16(sr qr)) (one
        // fused multiply-add, one rounding) XOR fp16(s q), so that one XOR
        // turns the widened weight into the patched one. Column c of the
        // lane's 32 sits in dword lane / 16 of lane r + 16 (c / 8) of the
        // tile, at nibble nib_pos(c % 8).
        const uint32_t dw = tw[(r + 16 * (c >> 3)) * 4 + (lane >> 4)];
        const int q = (int)((dw >> (4 * nib_pos(c & 7))) & 0xFu) - 8;
        const _Float16 wv = (_Float16)fmaf(sbase, (float)q, (float)dh);
        const _Float16 wb = (_Float16)(sbase * (float)q);
        wpatch[ps] = ((uint32_t)(__builtin_bit_cast(uint16_t, wv) ^ __builtin_bit_cast(uint16_t, wb)) << 16) |
                     ((uint32_t)r << 12) | kPatchValid | ((uint32_t)j & (kTileCols - 1));
        ++pc;
        ++ps;
      }
    }
    csr += sel_tot;
  }
}

// Canonical base codes [N][K/2] from the tile layout: one thread per 32
// columns, which sit in dword (c0 % 128) / 32 of the row's four lanes.
__global__ __launch_bounds__(256) void k_export_codes(const uint8_t* __restrict__ tiles, int N, int K, int Kt,
                                                      uint8_t* __restrict__ codes) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (row, 32-column chunk)
  const int chunks = K / 32;
  if (idx >= (int64_t)N * chunks) return;
  const int row = (int)(idx / chunks), ch = (int)(idx - (idx / chunks) * chunks);
  const int c0 = ch * 32;
  const int rb = row / kRowsPerBlock, kt = c0 / kTileCols, seg = (c0 % kTileCols) / 32;
  const uint32_t* tw = reinterpret_cast<const uint32_t*>(tiles) + ((int64_t)rb * Kt + kt) * (kWave * 4);
  uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t dw = tw[(row % kRowsPerBlock + 16 * g) * 4 + seg];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t u = (dw >> (4 * nib_pos(c))) & 0xFu;
      const int cc = 8 * g + c;               // column within the 32-column chunk
      o[cc >> 3] |= u << (4 * (cc & 7));      // canonical: column 2b low nibble, 2b+1 high
    }
  }
  reinterpret_cast<uint4*>(codes + (int64_t)row * (K / 2) + c0 / 2)[0] = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

// ------------------------------------------------------------------ host
#define MQ_TRY(x)                        \
  do {                                   \
    hipError_t err_ = (x);               \
    if (err_ != hipSuccess) return err_; \
  } while (0)

namespace {
struct Temp {
  void* p = nullptr;
  ~Temp() {
    if (p) (void)hipFree(p);
  }
};
}  // namespace

hipError_t pack_on_device(const uint16_t* W, mq_packed* p, hipStream_t stream, uint32_t* flags_out) {
  const int N = (int)p->N, K = (int)p->K, G = p->G;
  const int Kt = (int)p->Kt, Nb = (int)p->Nb;
  const int64_t ntiles = (int64_t)Nb * Kt;
  Temp t_state, t_hist, t_gt, t_eq, t_eb, t_rt, t_tc, t_dense;
  uint32_t* dense = nullptr;   // the dense row blocks (set when the stream is built)
  MQ_TRY(hipMalloc(&t_state.p, sizeof(SelState)));
  SelState* st = static_cast<SelState*>(t_state.p);
  SelState init{0ull, (uint64_t)p->nnz, 0u, 0u};
  MQ_TRY(hipMemcpyAsync(st, &init, sizeof(init), hipMemcpyHostToDevice, stream));
  MQ_TRY(hipMemsetAsync(p->scales, 0, (size_t)Nb * kRowsPerBlock * p->sstride * sizeof(uint16_t), stream));
  MQ_TRY(hipMemsetAsync(p->rscale, 0, (size_t)N * sizeof(float), stream));
  MQ_TRY(hipMemsetAsync(p->row_ptr, 0, (size_t)(N + 1) * sizeof(int32_t), stream));
  MQ_TRY(hipMemsetAsync(p->tile_ptr, 0, (size_t)(ntiles + 1) * sizeof(uint32_t), stream));
  MQ_TRY(hipMemsetAsync(p->entries, 0, (size_t)(p->stream_cap + kEntryPad) * sizeof(uint32_t), stream));
  MQ_TRY(hipMemsetAsync(p->wpatch, 0, (size_t)(p->stream_cap + kEntryPad) * sizeof(uint32_t), stream));

  k_pack_base<<<dim3((unsigned)ntiles), dim3(kWave), 0, stream>>>(W, N, K, G, Kt, p->sstride, p->tiles,
                                                                 p->scales, st);
  MQ_TRY(hipGetLastError());

  if (p->nnz > 0) {
    const size_t rc_bytes = (size_t)((p->nnz + 1) / 2 + 3) / 4 * 4;
    MQ_TRY(hipMemsetAsync(p->rcodes, 0, rc_bytes, stream));
    MQ_TRY(hipMalloc(&t_hist.p, kDigitBins * sizeof(uint32_t)));
    MQ_TRY(hipMemsetAsync(t_hist.p, 0, kDigitBins * sizeof(uint32_t), stream));
    uint32_t* hist = static_cast<uint32_t*>(t_hist.p);
    const int hist_blocks = (int)std::min<int64_t>(2048, (ntiles + 3) / 4);
    for (int pass = 0; pass < kDigitPasses; ++pass) {
      k_hist<<<dim3(hist_blocks), dim3(256), 0, stream>>>(W, p->scales, N, K, G, Kt, p->sstride, (int)ntiles,
                                                          pass, st, hist);
      MQ_TRY(hipGetLastError());
      k_select_digit<<<dim3(1), dim3(1024), 0, stream>>>(hist, st, pass);
      MQ_TRY(hipGetLastError());
    }
    MQ_TRY(hipMalloc(&t_gt.p, (size_t)N * sizeof(uint32_t)));
    MQ_TRY(hipMalloc(&t_eq.p, (size_t)N * sizeof(uint32_t)));
    MQ_TRY(hipMalloc(&t_eb.p, (size_t)N * sizeof(uint32_t)));
    MQ_TRY(hipMalloc(&t_rt.p, (size_t)N * Kt * sizeof(uint32_t)));
    MQ_TRY(hipMalloc(&t_tc.p, (size_t)ntiles * sizeof(uint32_t)));
    uint32_t* cgt = static_cast<uint32_t*>(t_gt.p);
    uint32_t* ceq = static_cast<uint32_t*>(t_eq.p);
    uint32_t* eb = static_cast<uint32_t*>(t_eb.p);
    uint32_t* crt = static_cast<uint32_t*>(t_rt.p);
    uint32_t* tcnt = static_cast<uint32_t*>(t_tc.p);
    k_row_counts<<<dim3(Nb), dim3(kWave), 0, stream>>>(W, p->scales, N, K, G, Kt, p->sstride, st, cgt, ceq);
    MQ_TRY(hipGetLastError());
    k_scan_rows<<<dim3(1), dim3(1024), 0, stream>>>(cgt, ceq, N, st, eb, p->row_ptr, (uint64_t)p->nnz);
    MQ_TRY(hipGetLastError());
    k_row_select<<<dim3(Nb), dim3(kWave), 0, stream>>>(W, p->scales, N, K, G, Kt, p->sstride, st, eb, p->rscale,
                                                       crt, tcnt);
    MQ_TRY(hipGetLastError());
    MQ_TRY(hipMalloc(&t_dense.p, 3 * kDenseListMax * sizeof(uint32_t)));
    dense = static_cast<uint32_t*>(t_dense.p);
    k_scan_tiles<<<dim3(1), dim3(1024), 0, stream>>>(tcnt, ntiles, p->Kt, p->tile_ptr, dense, st);
    MQ_TRY(hipGetLastError());
    k_row_emit<<<dim3(Nb), dim3(kWave), 0, stream>>>(W, p->scales, N, K, G, Kt, p->sstride, st, eb, p->row_ptr,
                                                     p->rscale, crt, p->tile_ptr, p->tiles, p->col,
                                                     reinterpret_cast<uint32_t*>(p->rcodes), p->entries, p->wpatch,
                                                     p->nnz,
                                                     p->stream_cap, st);
    MQ_TRY(hipGetLastError());
  }
  SelState fin;
  uint32_t nstream = 0;
  MQ_TRY(hipMemcpyAsync(&fin, st, sizeof(fin), hipMemcpyDeviceToHost, stream));
  MQ_TRY(hipMemcpyAsync(&nstream, p->tile_ptr + ntiles, sizeof(nstream), hipMemcpyDeviceToHost, stream));
  p->ndense = 0;
  if (dense) {
    MQ_TRY(hipStreamSynchronize(stream));
    p->ndense = fin.ndense;
    if (fin.ndense > 0 && fin.ndense <= (uint32_t)kDenseListMax) {
      uint32_t* dst[3] = {p->dense_rb, p->dense_e0, p->dense_nch};
      for (int a = 0; a < 3; ++a)
        MQ_TRY(hipMemcpyAsync(dst[a], dense + a * kDenseListMax, fin.ndense * sizeof(uint32_t),
                              hipMemcpyDeviceToHost, stream));
    }
  }
  MQ_TRY(hipStreamSynchronize(stream));
  *flags_out = fin.flags;
  p->nstream = nstream;
  p->max_seg = fin.max_seg;
  p->max_rb = fin.max_rb;
  if ((int64_t)nstream > p->stream_cap) *flags_out |= kFlagCountMismatch;
  return hipSuccess;
}

hipError_t launch_pack_base(const uint16_t* W, mq_packed* p, SelState* st, hipStream_t stream) {
  const int64_t ntiles = p->Nb * p->Kt;
  k_pack_base<<<dim3((unsigned)ntiles), dim3(kWave), 0, stream>>>(W, (int)p->N, (int)p->K, p->G, (int)p->Kt,
                                                                 p->sstride, p->tiles, p->scales, st);
  return hipGetLastError();
}

hipError_t launch_scan_tiles(const uint32_t* tile_cnt, int64_t ntiles, int64_t Kt, uint32_t* tile_ptr,
                             uint32_t* dense_rb, SelState* st, hipStream_t stream) {
  k_scan_tiles<<<dim3(1), dim3(1024), 0, stream>>>(tile_cnt, ntiles, Kt, tile_ptr, dense_rb, st);
  return hipGetLastError();
}

hipError_t export_tile_codes(const uint8_t* tiles, int64_t N, int64_t K, uint8_t* codes, hipStream_t stream) {
  const int64_t n = N * (K / 32);
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  k_export_codes<<<dim3(blocks), dim3(256), 0, stream>>>(tiles, (int)N, (int)K, (int)((K + kTileCols - 1) / kTileCols),
                                                          codes);
  return hipGetLastError();
}

hipError_t export_codes(const mq_packed* p, uint8_t* codes, hipStream_t stream) {
  return export_tile_codes(p->tiles, p->N, p->K, codes, stream);
}

}  // namespace mq
