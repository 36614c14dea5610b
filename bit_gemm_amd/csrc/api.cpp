// Host side of the C ABI: argument validation, the packed-layer handle, and
// dispatch to the HIP kernels. No kernel code lives here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>
#include <vector>

#include "mq_internal.h"
#include "gemv_group.h"

#define MQ_API extern "C" __attribute__((visibility("default")))

namespace {

std::mutex g_mu;
std::unordered_set<const mq_packed*> g_live;   // handles returned by mq_pack and not yet freed

bool is_live(const mq_packed* p) {
  if (!p) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  return g_live.count(p) != 0 && p->magic == mq::kMagic;
}

mq_status from_hip(hipError_t e) {
  if (e == hipSuccess) return MQ_OK;
  if (e == hipErrorOutOfMemory) return MQ_ERR_OUT_OF_MEMORY;
  return MQ_ERR_DEVICE;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

void release(mq_packed* p) {
  void* bufs[] = {p->tiles,    p->scales,  p->row_ptr, p->col,    p->rcodes, p->rscale,  p->tile_ptr,
                  p->entries, p->wpatch,  p->blk,     p->bscale, p->rt_ptr, p->rt_tiles,
                  p->rt_slot};
  for (void* b : bufs)
    if (b) (void)hipFree(b);
  p->magic = 0;
  delete p;
}

}  // namespace

MQ_API const char* mq_status_string(mq_status s) {
  switch (s) {
    case MQ_OK: return "MQ_OK";
    case MQ_ERR_INVALID_ARG: return "MQ_ERR_INVALID_ARG";
    case MQ_ERR_UNSUPPORTED: return "MQ_ERR_UNSUPPORTED";
    case MQ_ERR_NONFINITE: return "MQ_ERR_NONFINITE";
    case MQ_ERR_OUT_OF_MEMORY: return "MQ_ERR_OUT_OF_MEMORY";
    case MQ_ERR_DEVICE: return "MQ_ERR_DEVICE";
    case MQ_ERR_BAD_HANDLE: return "MQ_ERR_BAD_HANDLE";
  }
  return "MQ_ERR_UNKNOWN";
}

MQ_API mq_status mq_pack(const void* W_dev_fp16, int64_t N, int64_t K, int32_t group_size,
                         double residual_density, void* hip_stream, mq_packed** out) {
  if (out) *out = nullptr;
  if (!W_dev_fp16 || !out) return MQ_ERR_INVALID_ARG;
  if (N <= 0 || K <= 0) return MQ_ERR_INVALID_ARG;
  if (!(residual_density >= 0.0 && residual_density <= 1.0)) return MQ_ERR_INVALID_ARG;   // NaN fails too
  if (group_size != 32 && group_size != 64 && group_size != 128) return MQ_ERR_UNSUPPORTED;
  if (K % group_size != 0) return MQ_ERR_INVALID_ARG;
  if (K > 65536) return MQ_ERR_UNSUPPORTED;
  if (N >= (int64_t(1) << 31) / K) return MQ_ERR_UNSUPPORTED;   // N * K < 2^31
  if ((reinterpret_cast<uintptr_t>(W_dev_fp16) & 15u) != 0) return MQ_ERR_INVALID_ARG;

  const int64_t nk = N * K;
  int64_t nnz = (int64_t)std::floor(residual_density * (double)nk);   // one float64 product, then floor
  if (nnz > nk) nnz = nk;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return MQ_ERR_DEVICE;

  mq_packed* p = new (std::nothrow) mq_packed();
  if (!p) return MQ_ERR_OUT_OF_MEMORY;
  std::memset(p, 0, sizeof(*p));
  p->N = N;
  p->K = K;
  p->G = group_size;
  p->rho = residual_density;
  p->nnz = nnz;
  p->Nb = ceil_div(N, mq::kRowsPerBlock);
  p->Kt = ceil_div(K, mq::kTileCols);
  p->sstride = round_up(p->Kt * mq::kTileCols / group_size, 8);
  p->device = dev;

  const size_t n_tiles = (size_t)(p->Nb * p->Kt);
  const size_t sz_tiles = n_tiles * mq::kTileBytes;
  const size_t sz_scales = (size_t)(p->Nb * mq::kRowsPerBlock * p->sstride) * sizeof(uint16_t);
  const size_t sz_rowptr = (size_t)(N + 1) * sizeof(int32_t);
  const size_t sz_col = (size_t)std::max<int64_t>(nnz, 1) * sizeof(uint16_t);
  const size_t sz_rcodes = (size_t)round_up((nnz + 1) / 2 + 1, 4);
  const size_t sz_rscale = (size_t)N * sizeof(float);
  const size_t sz_tptr = (n_tiles + 1) * sizeof(uint32_t);
  // the stream pads each row block to a multiple of 32 entries and is
  // followed by zero entries so kernels may read whole chunks past its end
  p->stream_cap = nnz + (int64_t)(mq::kChunk - 1) * p->Nb;
  const size_t sz_ent = (size_t)(p->stream_cap + mq::kEntryPad) * sizeof(uint32_t);
  struct {
    void** dst;
    size_t n;
  } allocs[] = {{(void**)&p->tiles, sz_tiles},   {(void**)&p->scales, sz_scales}, {(void**)&p->row_ptr, sz_rowptr},
                {(void**)&p->col, sz_col},       {(void**)&p->rcodes, sz_rcodes}, {(void**)&p->rscale, sz_rscale},
                {(void**)&p->tile_ptr, sz_tptr}, {(void**)&p->entries, sz_ent},  {(void**)&p->wpatch, sz_ent}};
  size_t total = 0;
  for (auto& a : allocs) {
    e = hipMalloc(a.dst, a.n);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      release(p);
      return e == hipErrorOutOfMemory ? MQ_ERR_OUT_OF_MEMORY : MQ_ERR_DEVICE;
    }
    total += a.n;
  }
  p->bytes = total;

  uint32_t flags = 0;
  e = mq::pack_on_device(static_cast<const uint16_t*>(W_dev_fp16), p, static_cast<hipStream_t>(hip_stream), &flags);
  if (e != hipSuccess) {
    release(p);
    return from_hip(e);
  }
  if (flags & mq::kFlagNonFinite) {
    release(p);
    return MQ_ERR_NONFINITE;
  }
  if (flags & mq::kFlagScaleOverflow) {
    release(p);
    return MQ_ERR_UNSUPPORTED;
  }
  if (flags & mq::kFlagCountMismatch) {   // internal consistency check of the selection
    release(p);
    return MQ_ERR_DEVICE;
  }
  p->magic = mq::kMagic;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.insert(p);
  }
  *out = p;
  return MQ_OK;
}

static mq_status linear_impl(const void* X, int64_t M, const mq_packed* p, void* Y, void* stream, int32_t kernel) {
  if (!is_live(p)) return MQ_ERR_BAD_HANDLE;
  if (!X || !Y || M <= 0) return MQ_ERR_INVALID_ARG;
  if (M > (int64_t(1) << 31) / p->K || M > (int64_t(1) << 31) / p->N) return MQ_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(X) & 15u) != 0 || (reinterpret_cast<uintptr_t>(Y) & 7u) != 0)
    return MQ_ERR_INVALID_ARG;
  if (kernel < MQ_KERNEL_AUTO || kernel > MQ_KERNEL_GEMM) return MQ_ERR_INVALID_ARG;
  bool gemv;
  if (kernel == MQ_KERNEL_AUTO)
    gemv = mq::auto_gemv(p, M);
  else if (kernel == MQ_KERNEL_GEMV) {
    if (M > mq::kGemvMaxM) return MQ_ERR_UNSUPPORTED;
    gemv = true;
  } else
    gemv = false;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = gemv ? mq::launch_gemv(p, static_cast<const uint16_t*>(X), M, static_cast<uint16_t*>(Y), s)
                            : mq::launch_gemm(p, static_cast<const uint16_t*>(X), M, static_cast<uint16_t*>(Y), s);
  return from_hip(e);
}

MQ_API mq_status mq_pack_blocks(const void* W_dev_fp16, int64_t N, int64_t K, int32_t group_size,
                                double block_fraction, const float* h_dev_f32, void* hip_stream, mq_packed** out) {
  if (out) *out = nullptr;
  if (!W_dev_fp16 || !h_dev_f32 || !out) return MQ_ERR_INVALID_ARG;
  if (N <= 0 || K <= 0) return MQ_ERR_INVALID_ARG;
  if (!(block_fraction >= 0.0 && block_fraction <= 1.0)) return MQ_ERR_INVALID_ARG;   // NaN fails too
  if (group_size != 32 && group_size != 64 && group_size != 128) return MQ_ERR_UNSUPPORTED;
  if (K % group_size != 0) return MQ_ERR_INVALID_ARG;
  if (K > 65536) return MQ_ERR_UNSUPPORTED;
  if (N >= (int64_t(1) << 31) / K) return MQ_ERR_UNSUPPORTED;   // N * K < 2^31
  if ((reinterpret_cast<uintptr_t>(W_dev_fp16) & 15u) != 0 || (reinterpret_cast<uintptr_t>(h_dev_f32) & 3u) != 0)
    return MQ_ERR_INVALID_ARG;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return MQ_ERR_DEVICE;
  mq_packed* p = new (std::nothrow) mq_packed();
  if (!p) return MQ_ERR_OUT_OF_MEMORY;
  std::memset(p, 0, sizeof(*p));
  p->N = N;
  p->K = K;
  p->G = group_size;
  p->rho = block_fraction;
  p->Nb = ceil_div(N, mq::kRowsPerBlock);
  p->Kt = ceil_div(K, mq::kTileCols);
  p->sstride = round_up(p->Kt * mq::kTileCols / group_size, 8);
  p->device = dev;
  p->blocks = 1;
  const int64_t nblocks = p->Nb * p->Kt;
  int64_t nsel = (int64_t)std::floor(block_fraction * (double)nblocks);   // one float64 product, then floor
  if (nsel > nblocks) nsel = nblocks;
  p->nblk = nsel;

  // The handle holds what the kernels read: base tiles and scales, and the
  // residual blocks as code tiles with a scale per row, located by the
  // blocks' slot per tile and first block per row block. (The canonical
  // block codes are derived from the code tiles on export.)
  const size_t n_tiles = (size_t)nblocks;
  const size_t nb1 = (size_t)nsel + 1;   // one more all-zero block slot
  struct {
    void** dst;
    size_t n;
  } allocs[] = {{(void**)&p->tiles, n_tiles * mq::kTileBytes},
                {(void**)&p->scales, (size_t)(p->Nb * mq::kRowsPerBlock * p->sstride) * sizeof(uint16_t)},
                {(void**)&p->blk, nb1 * sizeof(int32_t)},
                {(void**)&p->bscale, nb1 * mq::kRowsPerBlock * sizeof(float)},
                {(void**)&p->rt_ptr, (size_t)(p->Nb + 1) * sizeof(uint32_t)},
                {(void**)&p->rt_tiles, nb1 * mq::kTileBytes},
                {(void**)&p->rt_slot, n_tiles * sizeof(int32_t)}};
  size_t total = 0;
  for (auto& a : allocs) {
    e = hipMalloc(a.dst, a.n);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      release(p);
      return e == hipErrorOutOfMemory ? MQ_ERR_OUT_OF_MEMORY : MQ_ERR_DEVICE;
    }
    total += a.n;
  }
  p->bytes = total;

  uint32_t flags = 0;
  e = mq::pack_blocks_on_device(static_cast<const uint16_t*>(W_dev_fp16), h_dev_f32, p,
                                static_cast<hipStream_t>(hip_stream), &flags);
  if (e != hipSuccess) {
    release(p);
    return from_hip(e);
  }
  mq_status st = MQ_OK;
  if (flags & mq::kFlagNonFinite) st = MQ_ERR_NONFINITE;
  else if (flags & mq::kFlagBadHessian) st = MQ_ERR_INVALID_ARG;
  else if (flags & mq::kFlagScaleOverflow) st = MQ_ERR_UNSUPPORTED;
  else if (flags & mq::kFlagCountMismatch) st = MQ_ERR_DEVICE;
  if (st != MQ_OK) {
    release(p);
    return st;
  }
  p->magic = mq::kMagic;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.insert(p);
  }
  *out = p;
  return MQ_OK;
}

MQ_API mq_status mq_block_count(const mq_packed* p, int64_t* nblk) {
  if (!is_live(p)) return MQ_ERR_BAD_HANDLE;
  if (!nblk) return MQ_ERR_INVALID_ARG;
  *nblk = p->blocks ? p->nblk : -1;
  return MQ_OK;
}

MQ_API mq_status mq_export_blocks(const mq_packed* p, void* blk_i32, void* rscale_f32, void* rcodes_u8,
                                  void* hip_stream) {
  if (!is_live(p)) return MQ_ERR_BAD_HANDLE;
  if (!p->blocks) return MQ_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const size_t n = (size_t)p->nblk;
  hipError_t e = hipSuccess;
  if (n == 0) return MQ_OK;
  if (blk_i32) e = hipMemcpyAsync(blk_i32, p->blk, n * sizeof(int32_t), hipMemcpyDefault, s);
  if (e == hipSuccess && rscale_f32)
    e = hipMemcpyAsync(rscale_f32, p->bscale, n * mq::kRowsPerBlock * sizeof(float), hipMemcpyDefault, s);
  if (e == hipSuccess && rcodes_u8)   // block n as a 16-row, 128-column layer of one tile per row block
    e = mq::export_tile_codes(p->rt_tiles, (int64_t)n * mq::kRowsPerBlock, mq::kTileCols,
                              static_cast<uint8_t*>(rcodes_u8), s);
  return from_hip(e);
}

MQ_API mq_status mq_smooth_weights(const void* W_dev_fp16, int64_t N, int64_t K, const float* amax_x_dev_f32,
                                   void* W_out_dev_fp16, int32_t* e_out_dev_i32, void* hip_stream) {
  if (!W_dev_fp16 || !amax_x_dev_f32 || !W_out_dev_fp16 || !e_out_dev_i32) return MQ_ERR_INVALID_ARG;
  if (N <= 0 || K <= 0) return MQ_ERR_INVALID_ARG;
  if (N >= (int64_t(1) << 31) / K) return MQ_ERR_UNSUPPORTED;   // N * K < 2^31
  if ((reinterpret_cast<uintptr_t>(W_dev_fp16) & 1u) || (reinterpret_cast<uintptr_t>(W_out_dev_fp16) & 1u) ||
      (reinterpret_cast<uintptr_t>(amax_x_dev_f32) & 3u) || (reinterpret_cast<uintptr_t>(e_out_dev_i32) & 3u))
    return MQ_ERR_INVALID_ARG;
  uint32_t flags = 0;
  const hipError_t e = mq::smooth_weights(static_cast<const uint16_t*>(W_dev_fp16), N, K, amax_x_dev_f32,
                                          static_cast<uint16_t*>(W_out_dev_fp16), e_out_dev_i32,
                                          static_cast<hipStream_t>(hip_stream), &flags);
  if (e != hipSuccess) return from_hip(e);
  return flags ? MQ_ERR_INVALID_ARG : MQ_OK;
}

MQ_API mq_status mq_smooth_activations(const void* X_dev_fp16, int64_t M, int64_t K, const int32_t* e_dev_i32,
                                       void* X_out_dev_fp16, void* hip_stream) {
  if (!X_dev_fp16 || !e_dev_i32 || !X_out_dev_fp16) return MQ_ERR_INVALID_ARG;
  if (M <= 0 || K <= 0) return MQ_ERR_INVALID_ARG;
  if (M >= (int64_t(1) << 31) / K) return MQ_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(X_dev_fp16) & 1u) || (reinterpret_cast<uintptr_t>(X_out_dev_fp16) & 1u) ||
      (reinterpret_cast<uintptr_t>(e_dev_i32) & 3u))
    return MQ_ERR_INVALID_ARG;
  return from_hip(mq::smooth_activations(static_cast<const uint16_t*>(X_dev_fp16), M, K, e_dev_i32,
                                         static_cast<uint16_t*>(X_out_dev_fp16), static_cast<hipStream_t>(hip_stream)));
}

MQ_API mq_status mq_linear(const void* X_dev_fp16, int64_t M, const mq_packed* p, void* Y_dev_fp16,
                           void* hip_stream) {
  return linear_impl(X_dev_fp16, M, p, Y_dev_fp16, hip_stream, MQ_KERNEL_AUTO);
}

MQ_API mq_status mq_linear_with(const void* X_dev_fp16, int64_t M, const mq_packed* p, void* Y_dev_fp16,
                                void* hip_stream, int32_t kernel) {
  return linear_impl(X_dev_fp16, M, p, Y_dev_fp16, hip_stream, kernel);
}

MQ_API mq_status mq_linear_noalloc(const void* X_dev_fp16, int64_t M, const mq_packed* p, void* Y_dev_fp16,
                                   void* hip_stream) {
  if (!is_live(p)) return MQ_ERR_BAD_HANDLE;
  if (!X_dev_fp16 || !Y_dev_fp16 || M <= 0) return MQ_ERR_INVALID_ARG;
  if (M > (int64_t(1) << 31) / p->K || M > (int64_t(1) << 31) / p->N) return MQ_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(X_dev_fp16) & 15u) != 0 || (reinterpret_cast<uintptr_t>(Y_dev_fp16) & 7u) != 0)
    return MQ_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const uint16_t* X = static_cast<const uint16_t*>(X_dev_fp16);
  uint16_t* Y = static_cast<uint16_t*>(Y_dev_fp16);
  if (mq::auto_gemv(p, M)) return from_hip(mq::launch_gemv(p, X, M, Y, s));   // no workspace on this path
  if (mq::gemm_workspace_bytes(p, M) > mq::gemm_scratch_capacity()) return MQ_ERR_UNSUPPORTED;
  return from_hip(mq::launch_gemm_noalloc(p, X, M, Y, s));
}

// n layers, each with its own input: one launch of the grouped decode kernel
// per run of up to kGroupMax layers that qualify, mq_linear for the others.
// Everything is validated before the first launch.
MQ_API mq_status mq_linear_group(const void* const* X_dev_fp16, int64_t M, const mq_packed* const* p,
                                 void* const* Y_dev_fp16, int32_t n, void* hip_stream) {
  if (!X_dev_fp16 || !p || !Y_dev_fp16 || n < 1 || M <= 0) return MQ_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    if (!is_live(p[i])) return MQ_ERR_BAD_HANDLE;
    if (!X_dev_fp16[i] || !Y_dev_fp16[i]) return MQ_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(X_dev_fp16[i]) & 15u) != 0 || (reinterpret_cast<uintptr_t>(Y_dev_fp16[i]) & 7u) != 0)
      return MQ_ERR_INVALID_ARG;
    if (M > (int64_t(1) << 31) / p[i]->K || M > (int64_t(1) << 31) / p[i]->N) return MQ_ERR_UNSUPPORTED;
  }
  // the layers that can share a launch (with the first such layer's group
  // size and device) go together, in runs of up to kGroupMax; the others run
  // on their own, as mq_linear would
  std::vector<const mq_packed*> gp;
  std::vector<const uint16_t*> gx;
  std::vector<uint16_t*> gy;
  std::vector<int32_t> solo;
  for (int32_t i = 0; i < n; ++i) {
    const bool fits = mq::gemv_group_takes(p + i, 1, M) &&
                      (gp.empty() || (p[i]->G == gp[0]->G && p[i]->device == gp[0]->device));
    if (fits) {
      gp.push_back(p[i]);
      gx.push_back(static_cast<const uint16_t*>(X_dev_fp16[i]));
      gy.push_back(static_cast<uint16_t*>(Y_dev_fp16[i]));
    } else {
      solo.push_back(i);
    }
  }
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int32_t ng = (int32_t)gp.size();
  for (int32_t i0 = 0; i0 < ng; i0 += mq::kGroupMax) {
    const mq_status st = from_hip(mq::launch_gemv_group(gp.data() + i0, gx.data() + i0, M, gy.data() + i0,
                                                        std::min<int32_t>(mq::kGroupMax, ng - i0), s));
    if (st != MQ_OK) return st;
  }
  for (const int32_t i : solo) {
    const mq_status st = linear_impl(X_dev_fp16[i], M, p[i], Y_dev_fp16[i], hip_stream, MQ_KERNEL_AUTO);
    if (st != MQ_OK) return st;
  }
  return MQ_OK;
}

// Row-wise concatenation of element-wise (or residual-free) handles; see
// include/mosaicq.h. Setup-time host code: the large arrays are copied device
// to device, the three whose values or nibble positions shift (row and tile
// pointers, residual codes) pass through host memory.
MQ_API mq_status mq_concat(const mq_packed* const* parts, int32_t n, void* hip_stream, mq_packed** out) {
  if (out) *out = nullptr;
  if (!parts || !out || n < 1) return MQ_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (!is_live(parts[i])) return MQ_ERR_BAD_HANDLE;
  const mq_packed* p0 = parts[0];
  int64_t N = 0, nnz = 0, nstream = 0;
  uint32_t max_seg = 0, max_rb = 0;
  uint64_t ndense = 0;
  for (int32_t i = 0; i < n; ++i) {
    const mq_packed* q = parts[i];
    if (q->blocks) return MQ_ERR_UNSUPPORTED;
    if (q->K != p0->K || q->G != p0->G || q->device != p0->device) return MQ_ERR_INVALID_ARG;
    // every part but the last fills its last row block, so output row r of
    // a part stays row r of its row blocks
    if (i + 1 < n && q->N % mq::kRowsPerBlock != 0) return MQ_ERR_INVALID_ARG;
    N += q->N;
    nnz += q->nnz;
    nstream += q->nstream;
    max_seg = std::max(max_seg, q->max_seg);
    max_rb = std::max(max_rb, q->max_rb);
    ndense += q->ndense;
  }
  const int64_t K = p0->K;
  if (N >= (int64_t(1) << 31) / K || nstream + mq::kEntryPad >= (int64_t(1) << 31)) return MQ_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MQ_ERR_DEVICE;
  if (dev != p0->device) return MQ_ERR_INVALID_ARG;

  mq_packed* p = new (std::nothrow) mq_packed();
  if (!p) return MQ_ERR_OUT_OF_MEMORY;
  std::memset(p, 0, sizeof(*p));
  p->N = N;
  p->K = K;
  p->G = p0->G;
  p->rho = (double)nnz / ((double)N * (double)K);
  p->nnz = nnz;
  p->Nb = ceil_div(N, mq::kRowsPerBlock);
  p->Kt = p0->Kt;
  p->sstride = p0->sstride;
  p->device = dev;
  p->max_seg = max_seg;
  p->max_rb = max_rb;
  p->nstream = nstream;
  p->stream_cap = nstream;   // the zero entries the kernels read past a segment start here
  const int64_t Kt = p->Kt;
  const size_t n_tiles = (size_t)(p->Nb * Kt);
  const size_t sz_rcodes = (size_t)round_up((nnz + 1) / 2 + 1, 4);
  const size_t sz_ent = (size_t)(nstream + mq::kEntryPad) * sizeof(uint32_t);
  struct {
    void** dst;
    size_t n;
  } allocs[] = {{(void**)&p->tiles, n_tiles * mq::kTileBytes},
                {(void**)&p->scales, (size_t)(p->Nb * mq::kRowsPerBlock * p->sstride) * sizeof(uint16_t)},
                {(void**)&p->row_ptr, (size_t)(N + 1) * sizeof(int32_t)},
                {(void**)&p->col, (size_t)std::max<int64_t>(nnz, 1) * sizeof(uint16_t)},
                {(void**)&p->rcodes, sz_rcodes},
                {(void**)&p->rscale, (size_t)N * sizeof(float)},
                {(void**)&p->tile_ptr, (n_tiles + 1) * sizeof(uint32_t)},
                {(void**)&p->entries, sz_ent},
                {(void**)&p->wpatch, sz_ent}};
  size_t total = 0;
  for (auto& a : allocs) {
    const hipError_t e = hipMalloc(a.dst, a.n);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      release(p);
      return e == hipErrorOutOfMemory ? MQ_ERR_OUT_OF_MEMORY : MQ_ERR_DEVICE;
    }
    total += a.n;
  }
  p->bytes = total;

  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  // host images of the shifted arrays
  int32_t* row_ptr = static_cast<int32_t*>(std::malloc((size_t)(N + 1) * sizeof(int32_t)));
  uint32_t* tile_ptr = static_cast<uint32_t*>(std::malloc((n_tiles + 1) * sizeof(uint32_t)));
  uint8_t* rcodes = static_cast<uint8_t*>(std::calloc(sz_rcodes, 1));
  size_t part_max = 1;
  for (int32_t i = 0; i < n; ++i)
    part_max = std::max({part_max, (size_t)(parts[i]->N + 1) * 4, (size_t)(parts[i]->Nb * Kt + 1) * 4,
                         (size_t)(parts[i]->nnz + 1) / 2 + 1});
  uint8_t* tmp = static_cast<uint8_t*>(std::malloc(part_max));
  hipError_t e = (row_ptr && tile_ptr && rcodes && tmp) ? hipSuccess : hipErrorOutOfMemory;
  if (e == hipSuccess) e = hipMemsetAsync(p->entries, 0, sz_ent, s);
  if (e == hipSuccess) e = hipMemsetAsync(p->wpatch, 0, sz_ent, s);
  int64_t rbo = 0, eo = 0, so = 0;
  for (int32_t i = 0; i < n && e == hipSuccess; ++i) {
    const mq_packed* q = parts[i];
    const int64_t ro = rbo * mq::kRowsPerBlock;
    e = hipMemcpyAsync(p->tiles + (size_t)(rbo * Kt) * mq::kTileBytes, q->tiles,
                       (size_t)(q->Nb * Kt) * mq::kTileBytes, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(p->scales + (size_t)(ro * p->sstride), q->scales,
                         (size_t)(q->Nb * mq::kRowsPerBlock * q->sstride) * sizeof(uint16_t), hipMemcpyDeviceToDevice,
                         s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(p->rscale + ro, q->rscale, (size_t)q->N * sizeof(float), hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && q->nnz > 0)
      e = hipMemcpyAsync(p->col + eo, q->col, (size_t)q->nnz * sizeof(uint16_t), hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && q->nstream > 0)
      e = hipMemcpyAsync(p->entries + so, q->entries, (size_t)q->nstream * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && q->nstream > 0)
      e = hipMemcpyAsync(p->wpatch + so, q->wpatch, (size_t)q->nstream * 4, hipMemcpyDeviceToDevice, s);
    // row pointers and tile pointers, shifted by the entries before this part
    if (e == hipSuccess) e = hipMemcpyAsync(tmp, q->row_ptr, (size_t)(q->N + 1) * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) {
      const int32_t* rp = reinterpret_cast<const int32_t*>(tmp);
      for (int64_t r = 0; r <= q->N; ++r) row_ptr[ro + r] = rp[r] + (int32_t)eo;
      e = hipMemcpyAsync(tmp, q->tile_ptr, (size_t)(q->Nb * Kt + 1) * 4, hipMemcpyDeviceToHost, s);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) {
      const uint32_t* tp = reinterpret_cast<const uint32_t*>(tmp);
      for (int64_t t = 0; t <= q->Nb * Kt; ++t) tile_ptr[rbo * Kt + t] = tp[t] + (uint32_t)so;
      if (q->nnz > 0) e = hipMemcpyAsync(tmp, q->rcodes, (size_t)(q->nnz + 1) / 2, hipMemcpyDeviceToHost, s);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) {   // entry t of the part is entry eo + t here: nibble (eo + t) & 1 of byte (eo + t) / 2
      for (int64_t t = 0; t < q->nnz; ++t) {
        const uint32_t u = (tmp[t >> 1] >> (4 * (t & 1))) & 0xFu;
        rcodes[(eo + t) >> 1] |= (uint8_t)(u << (4 * ((eo + t) & 1)));
      }
      // dense row blocks of this part, shifted (listed only while all fit)
      if (ndense <= (uint64_t)mq::kDenseListMax)
        for (uint32_t d = 0; d < q->ndense; ++d) {
          p->dense_rb[p->ndense] = q->dense_rb[d] + (uint32_t)rbo;
          p->dense_e0[p->ndense] = q->dense_e0[d] + (uint32_t)so;
          p->dense_nch[p->ndense] = q->dense_nch[d];
          ++p->ndense;
        }
    }
    rbo += q->Nb;
    eo += q->nnz;
    so += q->nstream;
  }
  p->ndense = (uint32_t)std::min<uint64_t>(ndense, 0xFFFFFFFFu);
  if (e == hipSuccess) e = hipMemcpyAsync(p->row_ptr, row_ptr, (size_t)(N + 1) * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(p->tile_ptr, tile_ptr, (n_tiles + 1) * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(p->rcodes, rcodes, sz_rcodes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);   // the host images are freed below
  std::free(row_ptr);
  std::free(tile_ptr);
  std::free(rcodes);
  std::free(tmp);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    release(p);
    return from_hip(e);
  }
  p->magic = mq::kMagic;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.insert(p);
  }
  *out = p;
  return MQ_OK;
}

MQ_API mq_status mq_residual_add(const void* X_dev_fp16, int64_t M, const mq_packed* p, void* Y_dev_fp16,
                                 void* hip_stream) {
  if (!is_live(p)) return MQ_ERR_BAD_HANDLE;
  if (!X_dev_fp16 || !Y_dev_fp16 || M <= 0) return MQ_ERR_INVALID_ARG;
  if (p->blocks) return MQ_ERR_UNSUPPORTED;   // it reads the element-wise CSR
  if (M > (int64_t(1) << 31) / p->K || M > (int64_t(1) << 31) / p->N) return MQ_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(X_dev_fp16) & 15u) != 0 || (reinterpret_cast<uintptr_t>(Y_dev_fp16) & 1u) != 0)
    return MQ_ERR_INVALID_ARG;
  return from_hip(mq::launch_residual(p, static_cast<const uint16_t*>(X_dev_fp16), M,
                                      static_cast<uint16_t*>(Y_dev_fp16), static_cast<hipStream_t>(hip_stream)));
}

MQ_API mq_status mq_quantize_activations(const void* X_dev_fp16, int64_t M, int64_t K, int32_t group_size,
                                         void* xq_dev_u8, void* xmeta_dev_u32, void* hip_stream) {
  if (!X_dev_fp16 || !xq_dev_u8 || !xmeta_dev_u32 || M <= 0 || K <= 0) return MQ_ERR_INVALID_ARG;
  if (group_size != 32 && group_size != 64 && group_size != 128) return MQ_ERR_INVALID_ARG;
  if (K % group_size != 0 || K > 65536) return MQ_ERR_INVALID_ARG;
  const int64_t Kp = ceil_div(K, mq::kTileCols) * mq::kTileCols;
  if (M >= (int64_t(1) << 31) / Kp) return MQ_ERR_UNSUPPORTED;   // M * Kp < 2^31
  if ((reinterpret_cast<uintptr_t>(X_dev_fp16) & 15u) || (reinterpret_cast<uintptr_t>(xq_dev_u8) & 15u) ||
      (reinterpret_cast<uintptr_t>(xmeta_dev_u32) & 3u))
    return MQ_ERR_INVALID_ARG;
  return from_hip(mq::quantize_a4(static_cast<const uint16_t*>(X_dev_fp16), M, K, group_size,
                                  static_cast<uint8_t*>(xq_dev_u8), static_cast<uint32_t*>(xmeta_dev_u32),
                                  static_cast<hipStream_t>(hip_stream)));
}

MQ_API mq_status mq_linear_a4(const void* xq_dev_u8, const void* xmeta_dev_u32, int64_t M, const mq_packed* p,
                              void* Y_dev_fp16, void* hip_stream) {
  if (!is_live(p)) return MQ_ERR_BAD_HANDLE;
  if (!xq_dev_u8 || !xmeta_dev_u32 || !Y_dev_fp16 || M <= 0) return MQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(xq_dev_u8) & 15u) || (reinterpret_cast<uintptr_t>(xmeta_dev_u32) & 3u) ||
      (reinterpret_cast<uintptr_t>(Y_dev_fp16) & 1u))
    return MQ_ERR_INVALID_ARG;
  // single residual entries carry their own scale, which the integer MFMA sum cannot take
  if (!p->blocks && p->nnz > 0) return MQ_ERR_UNSUPPORTED;
  const int64_t Kp = p->Kt * mq::kTileCols;
  if (M >= (int64_t(1) << 31) / Kp || M >= (int64_t(1) << 31) / p->N) return MQ_ERR_UNSUPPORTED;
  // the kernel addresses the handle's arrays with 32-bit byte offsets
  if (p->Nb * p->Kt * mq::kTileBytes >= (int64_t(1) << 31)) return MQ_ERR_UNSUPPORTED;
  return from_hip(mq::launch_gemm_a4(p, static_cast<const uint8_t*>(xq_dev_u8),
                                     static_cast<const uint32_t*>(xmeta_dev_u32), M,
                                     static_cast<uint16_t*>(Y_dev_fp16), static_cast<hipStream_t>(hip_stream)));
}

MQ_API mq_status mq_decode_a4(const void* X_dev_fp16, int64_t M, const mq_packed* p, void* Y_dev_fp16,
                              void* hip_stream) {
  if (!is_live(p)) return MQ_ERR_BAD_HANDLE;
  if (!X_dev_fp16 || !Y_dev_fp16 || M <= 0) return MQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(X_dev_fp16) & 15u) || (reinterpret_cast<uintptr_t>(Y_dev_fp16) & 1u))
    return MQ_ERR_INVALID_ARG;
  if (!p->blocks && p->nnz > 0) return MQ_ERR_UNSUPPORTED;   // as mq_linear_a4
  if (p->Nb * p->Kt * mq::kTileBytes >= (int64_t(1) << 31)) return MQ_ERR_UNSUPPORTED;
  if (!mq::decode_a4_fused_takes(p, M)) return MQ_ERR_UNSUPPORTED;
  return from_hip(mq::launch_decode_a4_fused(p, static_cast<const uint16_t*>(X_dev_fp16), M,
                                             static_cast<uint16_t*>(Y_dev_fp16), static_cast<hipStream_t>(hip_stream)));
}

MQ_API mq_status mq_stream_read(const void* src_dev, int64_t bytes, int32_t workgroups, void* sink_dev_u32,
                                void* hip_stream) {
  if (!src_dev || !sink_dev_u32 || bytes <= 0 || workgroups <= 0) return MQ_ERR_INVALID_ARG;
  if ((bytes & 15) != 0 || (reinterpret_cast<uintptr_t>(src_dev) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(sink_dev_u32) & 3u) != 0)
    return MQ_ERR_INVALID_ARG;
  if (bytes / 16 > (int64_t)workgroups * 256 * 16) return MQ_ERR_INVALID_ARG;   // at most 16 chunks per thread
  return from_hip(mq::stream_read(src_dev, bytes, workgroups, static_cast<uint32_t*>(sink_dev_u32),
                                  static_cast<hipStream_t>(hip_stream)));
}

MQ_API mq_status mq_packed_info(const mq_packed* p, int64_t* N, int64_t* K, int32_t* G, int64_t* nnz,
                                size_t* bytes) {
  if (!is_live(p)) return MQ_ERR_BAD_HANDLE;
  if (N) *N = p->N;
  if (K) *K = p->K;
  if (G) *G = p->G;
  if (nnz) *nnz = p->nnz;
  if (bytes) *bytes = p->bytes;
  return MQ_OK;
}

MQ_API mq_status mq_export_canonical(const mq_packed* p, void* codes_u8, void* scales_f16, void* row_ptr_i32,
                                     void* col_u16, void* rcodes_u8, void* rscale_f32, void* hip_stream) {
  if (!is_live(p)) return MQ_ERR_BAD_HANDLE;
  if (p->blocks && (row_ptr_i32 || col_u16 || rcodes_u8 || rscale_f32)) return MQ_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipError_t e = hipSuccess;
  if (codes_u8) {
    if ((reinterpret_cast<uintptr_t>(codes_u8) & 15u) != 0) return MQ_ERR_INVALID_ARG;
    e = mq::export_codes(p, static_cast<uint8_t*>(codes_u8), s);
    if (e != hipSuccess) return from_hip(e);
  }
  if (scales_f16) {
    e = hipMemcpy2DAsync(scales_f16, (size_t)(p->K / p->G) * 2, p->scales, (size_t)p->sstride * 2,
                         (size_t)(p->K / p->G) * 2, (size_t)p->N, hipMemcpyDefault, s);
    if (e != hipSuccess) return from_hip(e);
  }
  if (row_ptr_i32) {
    e = hipMemcpyAsync(row_ptr_i32, p->row_ptr, (size_t)(p->N + 1) * 4, hipMemcpyDefault, s);
    if (e != hipSuccess) return from_hip(e);
  }
  if (p->nnz > 0) {
    if (col_u16) {
      e = hipMemcpyAsync(col_u16, p->col, (size_t)p->nnz * 2, hipMemcpyDefault, s);
      if (e != hipSuccess) return from_hip(e);
    }
    if (rcodes_u8) {
      e = hipMemcpyAsync(rcodes_u8, p->rcodes, (size_t)(p->nnz + 1) / 2, hipMemcpyDefault, s);
      if (e != hipSuccess) return from_hip(e);
    }
  }
  if (rscale_f32) {
    e = hipMemcpyAsync(rscale_f32, p->rscale, (size_t)p->N * 4, hipMemcpyDefault, s);
    if (e != hipSuccess) return from_hip(e);
  }
  return MQ_OK;
}

MQ_API mq_status mq_export_tiled(const mq_packed* p, void* tiles_u8, void* tile_ptr_u32, void* entries_u32,
                                 void* hip_stream) {
  if (!is_live(p)) return MQ_ERR_BAD_HANDLE;
  if (p->blocks && (tile_ptr_u32 || entries_u32)) return MQ_ERR_UNSUPPORTED;   // no element-wise stream
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const size_t n_tiles = (size_t)(p->Nb * p->Kt);
  hipError_t e = hipSuccess;
  if (tiles_u8) e = hipMemcpyAsync(tiles_u8, p->tiles, n_tiles * mq::kTileBytes, hipMemcpyDefault, s);
  if (e == hipSuccess && tile_ptr_u32)
    e = hipMemcpyAsync(tile_ptr_u32, p->tile_ptr, (n_tiles + 1) * 4, hipMemcpyDefault, s);
  if (e == hipSuccess && entries_u32 && p->nstream > 0)
    e = hipMemcpyAsync(entries_u32, p->entries, (size_t)p->nstream * 4, hipMemcpyDefault, s);
  return from_hip(e);
}

MQ_API void mq_free(mq_packed* p) {
  if (!p) return;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_live.erase(p)) return;   // unknown or already freed: ignore
  }
  release(p);
}
