// Internal declarations shared by the host API and the HIP kernels of the
// packed 4-bit linear layer. Not part of the public ABI (see include/mosaicq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "../../include/mosaicq.h"

namespace mq {

// Geometry of the device layout.
constexpr int kRowsPerBlock = 16;   // rows of one code tile (one MFMA row block)
constexpr int kTileCols = 128;      // input columns of one code tile
constexpr int kTileBytes = 1024;    // 16 rows x 128 columns x 4 bits
constexpr int kColWindow = 4096;    // residual entries store column mod 4096
constexpr int kEntryPad = 1024;     // zero entries after the residual stream (read-ahead slack)
constexpr int kChunk = 32;          // residual entries per MFMA chunk; row-block segments are padded to it
constexpr int kDenseRbChunks = 16;  // row blocks with more chunks lead the dense-first decode order
constexpr int kDenseListMax = 64;   // dense row blocks a handle lists for the decode launch
constexpr uint32_t kPatchValid = 0x800u;   // bit 11 of a patched-weight entry (stream padding is 0)

struct Packed;  // layout of mq_packed (the opaque handle)

// Residual selection state, written by the radix passes on the device.
struct SelState {
  uint64_t prefix;   // bits of the threshold key found so far (key = bits of |e| as a double)
  uint64_t krem;     // entries still to take among keys equal to the current prefix
  uint32_t flags;    // kFlag* bits raised by the kernels
  uint32_t max_seg;  // the longest per-tile segment of the residual stream (entries, padding included)
  uint32_t max_rb;   // the longest row-block segment of the residual stream (entries, padding included)
  uint32_t ndense;   // row blocks with more than kDenseRbChunks chunks of the stream
};
constexpr uint32_t kFlagNonFinite = 1u;
constexpr uint32_t kFlagScaleOverflow = 2u;
constexpr uint32_t kFlagCountMismatch = 4u;
constexpr uint32_t kFlagBadHessian = 8u;   // a Hessian weight is negative or not finite

constexpr int kDigitBits = 13;                  // radix digit width of the top-k select
constexpr int kDigitBins = 1 << kDigitBits;
constexpr int kDigitPasses = 4;                 // digits at bits 51, 38, 25, 12 of the key
// keys are |e| * 2^24 < 2^41 stored as doubles: bits 0..11 are always zero

}  // namespace mq

struct mq_packed {
  uint64_t magic;
  int64_t N, K;
  int32_t G;
  double rho;
  int64_t nnz;
  int64_t Nb;       // row blocks = ceil(N / 16)
  int64_t Kt;       // column tiles = ceil(K / 128)
  int64_t sstride;  // scale row stride in elements
  int device;
  // device buffers (owned)
  uint8_t* tiles;       // [Nb][Kt][64][16] base codes
  uint16_t* scales;     // [Nb*16][sstride] fp16 bits
  int32_t* row_ptr;     // [N+1]
  uint16_t* col;        // [nnz]
  uint8_t* rcodes;      // [(nnz+1)/2 rounded up to 4]
  float* rscale;        // [N]
  uint32_t* tile_ptr;   // [Nb*Kt + 1] (element-wise handles)
  uint32_t* entries;    // [nstream + kEntryPad]: residual stream, row blocks padded to 32 entries (element-wise)
  uint32_t max_seg;     // the longest per-tile segment of the stream (entries, padding included)
  uint32_t max_rb;      // the longest row-block segment of the stream (entries, padding included)
  uint32_t* wpatch;     // [nstream + kEntryPad]: the same entries as patches of the GEMM kernels' widened
                        // weights: bits 0-6 column mod 128, 11 valid, 12-15 row mod 16, 16-31
                        // fp16(s q + fp16(sr qr)) XOR fp16(s q); element-wise handles only
  int64_t nstream;      // entries in the stream incl. the per-row-block zero padding
  int64_t stream_cap;   // allocated stream length (excluding the trailing zero pad)
  size_t bytes;
  // block-wise residual (mq_pack_blocks); the CSR fields above are unused then
  int32_t blocks;       // 1 for a handle from mq_pack_blocks
  int64_t nblk;         // selected 16 x 128 residual blocks
  int32_t* blk;         // [nblk] block indices rb * Kt + kt, ascending
  float* bscale;        // [nblk][16] residual scale of each block row
  uint32_t* rt_ptr;     // [Nb + 1]: the blocks of row block rb are blk[rt_ptr[rb] .. rt_ptr[rb + 1])
  uint8_t* rt_tiles;    // [nblk + 1][1 KiB]: the blocks' codes in the code-tile layout; slot nblk
                        // (like blk[nblk] = 0 and bscale[nblk][*] = 0) is an all-zero residual
  int32_t* rt_slot;     // [Nb * Kt]: the residual slot of each tile (nblk where it has none)
  // the row blocks with more than mq::kDenseRbChunks chunks of the stream, ascending (element-wise
  // handles; ndense > mq::kDenseListMax: too many to list, the decode launch keeps the plain order)
  uint32_t ndense;
  uint32_t dense_rb[mq::kDenseListMax];
  uint32_t dense_e0[mq::kDenseListMax];    // their first stream entries
  uint32_t dense_nch[mq::kDenseListMax];   // their chunks
};

namespace mq {

constexpr uint64_t kMagic = 0x4d6f736169635134ull;  // "MosaicQ4"

// Packing pipeline (pack.hip). Runs every kernel on `stream`; returns the
// first HIP error. Temporary buffers are allocated and freed inside.
hipError_t pack_on_device(const uint16_t* W, mq_packed* p, hipStream_t stream, uint32_t* flags_out);

// Block-wise packing (pack_blocks.hip): base as pack_on_device, then the
// nsel = p->nblk blocks with the largest Hessian-weighted score get their
// residual. h: [K] fp32 device weights.
hipError_t pack_blocks_on_device(const uint16_t* W, const float* h, mq_packed* p, hipStream_t stream,
                                 uint32_t* flags_out);

// Pieces of the element-wise pipeline the block packer reuses (pack.hip).
hipError_t launch_pack_base(const uint16_t* W, mq_packed* p, SelState* st, hipStream_t stream);
hipError_t launch_scan_tiles(const uint32_t* tile_cnt, int64_t ntiles, int64_t Kt, uint32_t* tile_ptr,
                             uint32_t* dense_rb, SelState* st,
                             hipStream_t stream);

// Outlier migration (migrate.hip): e_j and W^ = W 2^e (W_out may be W);
// synchronises; *flags_out != 0 when an activation maximum is negative or not
// finite.
hipError_t smooth_weights(const uint16_t* W, int64_t N, int64_t K, const float* amax_x, uint16_t* W_out,
                          int32_t* e_out, hipStream_t stream, uint32_t* flags_out);
// X^ = X 2^-e (X_out may be X); enqueued only.
hipError_t smooth_activations(const uint16_t* X, int64_t M, int64_t K, const int32_t* e, uint16_t* X_out,
                              hipStream_t stream);

// Canonical / tiled export (pack.hip).
hipError_t export_codes(const mq_packed* p, uint8_t* codes, hipStream_t stream);
// The same for any array of code tiles laid out as an N x K layer (tile
// (rb, kt) at (rb * ceil(K / 128) + kt) * 1 KiB; K a multiple of 32).
hipError_t export_tile_codes(const uint8_t* tiles, int64_t N, int64_t K, uint8_t* codes, hipStream_t stream);

// Decode kernel (gemv.hip): M <= 64 (block-residual handles with K != 4096
// or more than 16 tokens run the mid-size kernel).
hipError_t launch_gemv(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t stream);

// Prefill kernel (gemm.hip): any M >= 1 (up to 64 tokens it runs the
// mid-size kernel below).
hipError_t launch_gemm(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t stream);

// Prefill kernel with the weights widened in registers (gemm_rw.hip), for
// the handles and shapes gemm_rw_takes accepts.
bool gemm_rw_takes(const mq_packed* p, int64_t M);
hipError_t launch_gemm_rw(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t stream);

// Mid-size batch kernel (gemm_mid.hip): M <= 64, no workspace.
hipError_t launch_gemm_mid(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t stream);
constexpr int64_t kGemmMidMaxM = 64;

// mq_linear's GEMM path with the split-K partials in the library's static
// scratch array instead of a stream-ordered allocation (gemm.hip): no
// allocation at all. gemm_workspace_bytes: the partials' size for (p, M);
// gemm_scratch_capacity: the array's size.
hipError_t launch_gemm_noalloc(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t stream);
size_t gemm_workspace_bytes(const mq_packed* p, int64_t M);
size_t gemm_scratch_capacity();

// Separate residual kernel (residual.hip): Y <- fp16(Y + X R^T) from the
// canonical CSR, for the unfused comparison.
hipError_t launch_residual(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t stream);

// Y = fp16(sum of the S fp32 slices part[S][M][N]), slices added in order
// (gemm.hip); used by the kernels that split K.
hipError_t launch_splitk_reduce(const float* part, uint16_t* Y, int64_t M, int64_t N, int S, hipStream_t stream);

// 4-bit activations (w4a4.hip): the activation quantizer (codes in tile
// order, per-(token, group) scale and code sum), and the W4A4 GEMM.
hipError_t quantize_a4(const uint16_t* X, int64_t M, int64_t K, int G, uint8_t* xq, uint32_t* xmeta,
                       hipStream_t stream);
hipError_t launch_gemm_a4(const mq_packed* p, const uint8_t* xq, const uint32_t* xmeta, int64_t M, uint16_t* Y,
                          hipStream_t stream);
// The W4A4 decode kernel quantizing the fp16 activations itself (one
// kernel, no intermediate buffers), for the (p, M) decode_a4_fused_takes
// accepts: up to 2 tokens and K <= 4096.
bool decode_a4_fused_takes(const mq_packed* p, int64_t M);
hipError_t launch_decode_a4_fused(const mq_packed* p, const uint16_t* X, int64_t M, uint16_t* Y, hipStream_t stream);

// Streaming-read probe (probe.hip): reads bytes (a multiple of 16) of src
// with 16-byte loads, one XOR word per workgroup into sink[workgroups].
hipError_t stream_read(const void* src, int64_t bytes, int workgroups, uint32_t* sink, hipStream_t stream);

constexpr int64_t kGemvMaxM = 64;       // the GEMV kernels accept up to 64 tokens

// The automatic choice: the GEMV kernels up to 16 tokens when K <= 4096 (X
// whole in LDS), else up to 3 (with X from global memory they lose to the
// mid-size kernel from about 4 tokens on); the GEMM path (the mid-size kernel
// up to 64 tokens) otherwise.
inline bool auto_gemv(const mq_packed* p, int64_t M) { return M <= (p->K <= 4096 ? 16 : 3); }

}  // namespace mq
