/*
 * mosaicq.h -- C ABI of the MI355X (gfx950) fused "dense 4-bit base + sparse
 * 4-bit residual" linear layer.
 *
 * What is computed (MosaicQuant explainer, gist.science, Technical Summary,
 * Methodology section 1, Eq. (1); section 3 "ZipperEngine"):
 *   the weight W [N, K] (fp16, nn.Linear layout [out, in]) is split into a
 *   dense INT4 base Q(W) and a sparse INT4 residual R, and the layer computes
 *   Y = X (Q(W) + R)^T  with X [M, K] and Y [M, N] in fp16, fp32 accumulation,
 *   in one fused kernel per call.
 *
 * Quantiser (readings of the pages, which leave these details open):
 *   base     s[i,g] = fp16_rne(max_{j in group g} |W_ij| / 7), group = G
 *            consecutive input columns; q = clamp(rne(W/s), -7, 7) (0 if s = 0);
 *   error    e = W - s q (exact);
 *   residual the k = floor(rho N K) entries first in the order (|e| desc,
 *            row-major index asc) -- the Hessian-weighted block score of the
 *            pages' Methodology section 2 with an identity Hessian and 1x1
 *            blocks; per row sr_i = fp32_rne(max selected |e| / 7) and
 *            qr = clamp(rne(e/sr), -7, 7) (0 if sr = 0).
 *
 * Conventions for every entry point:
 *   - pointers named *_dev are device pointers on the device that is current
 *     when the call is made; W, X, Y must be contiguous row-major and 16-byte
 *     aligned; they stay owned by the caller;
 *   - hip_stream is a hipStream_t (NULL = the default stream); work is enqueued
 *     on it in order;
 *   - nothing throws across the ABI; each call returns an mq_status. Arguments
 *     are validated before any HIP call is made.
 */
#ifndef MOSAICQ_H
#define MOSAICQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mq_packed mq_packed; /* opaque; owns every device buffer of one packed layer */

typedef enum {
  MQ_OK = 0,
  MQ_ERR_INVALID_ARG = -1,   /* null pointer, size <= 0, K % G != 0, rho outside [0,1] or NaN */
  MQ_ERR_UNSUPPORTED = -2,   /* G not in {32,64,128}, K > 65536, N*K >= 2^31, a base scale whose
                                7*s overflows fp16, or a kernel choice that cannot run this M */
  MQ_ERR_NONFINITE = -3,     /* W holds Inf or NaN */
  MQ_ERR_OUT_OF_MEMORY = -4, /* a device allocation failed */
  MQ_ERR_DEVICE = -5,        /* a HIP call failed (no device, launch failure, fault seen at a sync) */
  MQ_ERR_BAD_HANDLE = -6     /* the handle is NULL, freed, or was never returned by mq_pack */
} mq_status;

/*
 * mq_pack -- disaggregate W into base codes, scales and the sparse residual
 * (Eq. (1) and the top-K allocation of Methodology section 2, read as above).
 *
 *   W_dev_fp16         [N, K] fp16 weights (device, caller-owned, read only)
 *   N, K               output / input features; K % group_size == 0, K <= 65536,
 *                      N * K < 2^31
 *   group_size         G in {32, 64, 128}
 *   residual_density   rho in [0, 1]; nnz = floor(rho * N * K) residual entries
 *   hip_stream         stream the packing kernels run on
 *   out                receives a new handle; *out is set to NULL on failure
 *
 * The packing runs entirely on the GPU and is deterministic: the packed
 * arrays are bit-identical run to run. The call synchronises hip_stream once
 * at the end (to report MQ_ERR_NONFINITE / MQ_ERR_UNSUPPORTED found on the
 * device), so it returns with the handle ready. Free it with mq_free.
 */
mq_status mq_pack(const void* W_dev_fp16, int64_t N, int64_t K, int32_t group_size,
                  double residual_density, void* hip_stream, mq_packed** out);

/*
 * mq_linear -- Y = X (deq(Q_base) + deq(R))^T for one packed layer
 * (ZipperEngine, Methodology section 3: the residual is applied inside the
 * dense 4-bit kernel, not by a second kernel).
 *
 *   X_dev_fp16   [M, K] fp16 activations (device, caller-owned)
 *   M            number of tokens, M >= 1
 *   p            handle from mq_pack (read only; calls on several streams may
 *                share it)
 *   Y_dev_fp16   [M, N] fp16 output (device, caller-owned, fully overwritten)
 *   hip_stream   stream to enqueue on; the call returns without synchronising
 *
 * Decode batches (up to 16 tokens with K <= 4096, up to 3 tokens for larger
 * K) run a GEMV-style kernel that streams the 4-bit tiles from HBM; up to 64
 * tokens a mid-size MFMA kernel that splits K among the waves of each
 * workgroup; above that the MFMA GEMM. All are deterministic. When the
 * GEMM's output tiles are too few to fill the GPU (M times N small against
 * K), it splits K across workgroups: the parts write fp32 partial sums to a
 * workspace that the call takes from the stream-ordered allocator
 * (hipMallocAsync / hipFreeAsync on hip_stream, so it also works under
 * stream capture, where it becomes a graph allocation), and a second kernel
 * adds the parts in a fixed order. The workspace holds at most
 * 256 x 256 x 256 fp32 values (64 MiB); if it cannot be allocated the call
 * returns MQ_ERR_OUT_OF_MEMORY. Up to 64 tokens no workspace is used.
 */
mq_status mq_linear(const void* X_dev_fp16, int64_t M, const mq_packed* p,
                    void* Y_dev_fp16, void* hip_stream);

/*
 * mq_linear_noalloc -- mq_linear for callers that cannot allocate device
 * memory during the call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, kernels, results (bit for
 * bit) and errors as mq_linear, but it allocates nothing: where mq_linear
 * splits K across workgroups (M > 64 on layers with fewer than 256 output
 * tiles) and takes the fp32 partial sums from a stream-ordered allocation,
 * this entry point puts them in a workspace array the library holds on each
 * GPU for the life of the process (64 MiB, set up on the first call on that
 * device). The split rule bounds the partials at 64 MiB, so every call fits;
 * a call that would need more returns MQ_ERR_UNSUPPORTED. All calls on one
 * GPU share that array: calls that overlap in time on one GPU (different
 * streams, or graphs replayed concurrently) race and must be ordered by the
 * caller. Every partial is written before it is read, so the array needs no
 * clearing between calls.
 */
mq_status mq_linear_noalloc(const void* X_dev_fp16, int64_t M, const mq_packed* p, void* Y_dev_fp16,
                            void* hip_stream);

/*
 * mq_linear_group -- mq_linear for n layers at once, each with its own input
 * (say the linears of one transformer block at decode): Y[i] = the fused
 * W4 + sparse-residual linear of X[i] with p[i] (MosaicQuant explainer,
 * Methodology section 3), each equal, bit for bit, to mq_linear(X[i], M, p[i],
 * Y[i]) on the same stream. Layers with K = 4096 and no block residual
 * (mq_pack_blocks), at 1 <= M <= 16 (for M <= 4 also: no row block of 16 rows
 * with more than 2560 residual entries), can share a launch:
 * the layers that meet these (with the group size and device of the first
 * of them) run in one kernel launch per 8 (from 5 tokens on, workgroups take
 * several row blocks of one layer, so the input is copied into LDS fewer
 * times; at any M the layers' ramps and tails overlap), and the others are
 * launched after them as mq_linear would.
 *
 *   X_dev_fp16   n pointers (host array) to [M, p[i]->K] fp16 inputs (device,
 *                16-byte aligned); inputs may be shared between layers
 *   M            tokens of every input, M > 0
 *   p            n live handles (host array)
 *   Y_dev_fp16   n pointers (host array) to [M, p[i]->N] fp16 outputs
 *                (device, 8-byte aligned, overwritten, not overlapping each
 *                other or any input)
 *   n            n >= 1
 *   hip_stream   stream to enqueue on (no synchronisation)
 *
 * Every argument is checked before anything is enqueued. Errors:
 * MQ_ERR_BAD_HANDLE, MQ_ERR_INVALID_ARG (NULL arrays or pointers, misaligned
 * pointers, M <= 0, n < 1), MQ_ERR_UNSUPPORTED (as mq_linear), MQ_ERR_DEVICE,
 * MQ_ERR_OUT_OF_MEMORY (a layer launched on its own whose GEMM needs a
 * workspace, as mq_linear).
 */
mq_status mq_linear_group(const void* const* X_dev_fp16, int64_t M, const mq_packed* const* p,
                          void* const* Y_dev_fp16, int32_t n, void* hip_stream);

/* Kernel choice for mq_linear_with. */
typedef enum { MQ_KERNEL_AUTO = 0, MQ_KERNEL_GEMV = 1, MQ_KERNEL_GEMM = 2 } mq_kernel;

/*
 * mq_linear_with -- mq_linear with the kernel chosen by the caller (tests and
 * benchmarks pin the dispatch with it). MQ_KERNEL_GEMV accepts M <= 64 and
 * returns MQ_ERR_UNSUPPORTED above that; MQ_KERNEL_GEMM accepts any M >= 1.
 */
mq_status mq_linear_with(const void* X_dev_fp16, int64_t M, const mq_packed* p,
                         void* Y_dev_fp16, void* hip_stream, int32_t kernel);

/*
 * mq_residual_add -- Y <- Y + X R^T with a separate kernel, R the sparse
 * residual of p (R_ij = sr_i * qr_ij on the selected entries, read from the
 * canonical CSR), accumulated in fp32 and rounded to fp16 into Y.
 *
 * This is the unfused two-kernel alternative the pages compare against
 * (MosaicQuant explainer, Methodology section 3: a separate residual kernel
 * must load the activations again and merge partial outputs). mq_linear on a
 * handle packed with residual_density 0 from the same W, followed by this
 * call on the handle with the residual, gives the unfused result of the same
 * layer; mq_linear itself never needs it. Built for the decode regime: a
 * workgroup stages a chunk of token rows of X in LDS (16 rows at K = 4096,
 * up to 64 for short K, 1 at K = 65536) and walks a range of CSR rows.
 *
 *   X_dev_fp16   [M, K] fp16 activations (device, caller-owned, 16-byte aligned)
 *   M            number of tokens, M >= 1
 *   p            handle from mq_pack (read only)
 *   Y_dev_fp16   [M, N] fp16 (device, caller-owned): read, updated in place;
 *                rows of W without residual entries leave Y unchanged
 *   hip_stream   stream to enqueue on; the call returns without synchronising
 *
 * Errors: MQ_ERR_BAD_HANDLE, MQ_ERR_INVALID_ARG (NULL pointers, M <= 0,
 * misaligned X), MQ_ERR_UNSUPPORTED (M * K or M * N >= 2^31), MQ_ERR_DEVICE.
 * A handle with nnz = 0 enqueues nothing.
 */
mq_status mq_residual_add(const void* X_dev_fp16, int64_t M, const mq_packed* p, void* Y_dev_fp16,
                          void* hip_stream);

/*
 * mq_packed_info -- sizes of a packed layer; any output pointer may be NULL.
 *   bytes = device bytes the handle owns: codes and scales, and for mq_pack
 *   the canonical residual and the two tile-ordered residual streams the
 *   kernels read, for mq_pack_blocks the residual blocks as code tiles.
 */
mq_status mq_packed_info(const mq_packed* p, int64_t* N, int64_t* K, int32_t* G,
                         int64_t* nnz, size_t* bytes);

/*
 * mq_export_canonical -- copy the packed layer out in the canonical layout
 * (all destinations are device buffers the caller allocated; any may be NULL
 * to skip it). Enqueued on hip_stream; synchronise before reading.
 *   codes_u8    [N, K/2]  base code u = q + 8; byte b of a row holds column 2b
 *                         in the low nibble and 2b+1 in the high nibble
 *   scales_f16  [N, K/G]  base scales
 *   row_ptr_i32 [N+1]     CSR row pointer of the residual
 *   col_u16     [nnz]     residual column, ascending within each row
 *   rcodes_u8   [(nnz+1)/2] residual code u = qr + 8, entry 2t in the low
 *                         nibble of byte t, 2t+1 in the high nibble; an unused
 *                         last high nibble is 0
 *   rscale_f32  [N]       residual row scale (0 for rows without entries)
 */
mq_status mq_export_canonical(const mq_packed* p, void* codes_u8, void* scales_f16,
                              void* row_ptr_i32, void* col_u16, void* rcodes_u8,
                              void* rscale_f32, void* hip_stream);

/*
 * mq_export_tiled -- copy out the device-side layout the kernels read (for
 * tests of the packer; any destination may be NULL). With Nb = ceil(N/16) row
 * blocks and Kt = ceil(K/128) column tiles:
 *   tiles_u8      [Nb, Kt, 64, 16]  1 KiB per (row block, tile): lane l owns
 *                 row 16*rb + (l % 16); its dword t (0..3) holds the 8 columns
 *                 128*kt + 32*t + 8*(l / 16) + c, c = 0..7, with column offset c
 *                 in nibble (c / 2) + 4 * (c % 2); padding holds code 8 (q = 0)
 *   tile_ptr_u32  [Nb * Kt + 1]     start of each (row block, tile) segment in
 *                 the residual stream; tile_ptr[Nb * Kt] is the stream length
 *   entries_u32   [tile_ptr[Nb*Kt]] residual stream sorted by (row block, tile,
 *                 row, column): bits 0-11 column mod 4096, bits 12-15 row mod 16,
 *                 bits 16-31 the residual value sr*qr rounded to fp16, which the
 *                 decode kernels add to the base weight s*q. Each row block's
 *                 segment ends with zero entries up to a multiple of 32. (The
 *                 mid-size and prefill kernels read a parallel copy of this
 *                 stream, not exported, whose entries hold the patched weight
 *                 fp16(s*q + that value) XOR fp16(s*q) instead.)
 * A handle from mq_pack_blocks has no residual stream: tile_ptr_u32 or
 * entries_u32 non-NULL return MQ_ERR_UNSUPPORTED for it (tiles_u8 works).
 */
mq_status mq_export_tiled(const mq_packed* p, void* tiles_u8, void* tile_ptr_u32,
                          void* entries_u32, void* hip_stream);

/*
 * mq_pack_blocks -- pack W with a block-wise residual chosen by a
 * Hessian-guided score (MosaicQuant explainer, Methodology section 2,
 * Block-Wise Residual Allocation: the budget goes to blocks; a Delta-score
 * weights each block's residual error with the diagonal Hessian estimate of
 * the input channels and approximates the drop of the output distortion;
 * the top-K blocks get a 4-bit residual).
 *
 * The base is exactly that of mq_pack. A block is one 16 x 128 tile (rows
 * 16 rb .., columns 128 kt ..; partial at the edges). For every block and
 * every row i of it: sr = fp32(max |e_ij| / 7) over the block's columns and
 * qr = clamp(rne(e / sr), -7, 7), e = w - s q the exact base error. The score
 * is Delta = sum, over the block's rows and then columns in ascending order,
 * of h_j * (r * (2 e - r)) with r = sr * qr, every operation rounded to
 * float64 (a fixed order, so the selection is reproducible); it equals the
 * drop of sum_j h_j (w - W~)^2 the block's residual brings. The
 * floor(block_fraction * number of blocks) blocks first in the order (Delta
 * descending, block index rb * ceil(K/128) + kt ascending) keep their
 * residual; the other entries keep the base only.
 *
 *   W_dev_fp16, N, K, group_size, hip_stream, out  as for mq_pack
 *   block_fraction  in [0, 1]
 *   h_dev_f32       [K] fp32 device weights of the input channels, >= 0 and
 *                   finite (for calibration activations X: h_j = sum_m X_mj^2);
 *                   read during the call only, 4-byte aligned
 *
 * The handle runs in mq_linear / mq_linear_with like any other. It holds the
 * selected blocks as 4-bit code tiles with a scale per row, which every
 * kernel widens like the base tiles (MQ_KERNEL_GEMV with K != 4096 or more
 * than 16 tokens runs the mid-size kernel for it), and nothing else of the
 * residual: about 1 KiB + 64 B per block on top of the plain handle.
 * mq_packed_info's nnz counts the blocks' nonzero residual codes.
 * mq_residual_add, the residual arrays of mq_export_canonical and the
 * residual stream of mq_export_tiled are not available for it
 * (MQ_ERR_UNSUPPORTED; codes and scales export as usual); mq_export_blocks
 * gives the residual. Synchronises hip_stream once, like
 * mq_pack. Errors as mq_pack, plus MQ_ERR_INVALID_ARG for block_fraction
 * outside [0, 1] (or NaN), a NULL or misaligned h, or a negative or
 * non-finite h value.
 */
mq_status mq_pack_blocks(const void* W_dev_fp16, int64_t N, int64_t K, int32_t group_size,
                         double block_fraction, const float* h_dev_f32, void* hip_stream,
                         mq_packed** out);

/* mq_block_count -- number of residual blocks of a handle from mq_pack_blocks
 * (-1 for a handle from mq_pack). */
mq_status mq_block_count(const mq_packed* p, int64_t* nblk);

/*
 * mq_export_blocks -- the block residual of a handle from mq_pack_blocks, in
 * canonical form (device destinations, any may be NULL; enqueued on
 * hip_stream). With B = mq_block_count:
 *   blk_i32     [B]           selected block indices rb * ceil(K/128) + kt, ascending
 *   rscale_f32  [B, 16]       residual scale of each block row (0 past row N - 1)
 *   rcodes_u8   [B, 16, 64]   residual code u = qr + 8 of each block row; byte b
 *                             holds column 2b in the low nibble and 2b+1 in the
 *                             high nibble; entries past the matrix hold 8
 * MQ_ERR_UNSUPPORTED for a handle from mq_pack.
 */
mq_status mq_export_blocks(const mq_packed* p, void* blk_i32, void* rscale_f32, void* rcodes_u8,
                           void* hip_stream);

/*
 * mq_smooth_weights -- move activation outliers into the weights before
 * packing (MosaicQuant explainer, Methodology section 1: an equivalent
 * transformation such as SmoothQuant migrates the activation outliers into
 * W, and the migrated matrix is what gets decomposed).
 *
 * SmoothQuant at strength 1/2 with power-of-two factors: for input channel
 * j, e_j = floor((E_x - E_w) / 2) where E_x = floor(log2 amax_x[j]) and
 * E_w = floor(log2 max_i |W_ij|) (from the floats' exponents); e_j = 0 when
 * either maximum is 0; e_j is clamped so that neither scaled maximum exceeds
 * fp16's range (exponent 15) and to [-24, 24]. Then W^_ij = fp16(W_ij 2^e_j),
 * exact unless the result is fp16-subnormal (round half to even). Pack W^ and
 * feed mq_linear activations from mq_smooth_activations: X^ W^^T = X W^T.
 *
 *   W_dev_fp16      [N, K] fp16 weights (device, 2-byte aligned)
 *   amax_x_dev_f32  [K] max |X_mj| per input channel over calibration
 *                   activations (device, >= 0 and finite)
 *   W_out_dev_fp16  [N, K] fp16 output W^ (device; may be W itself)
 *   e_out_dev_i32   [K] the exponents e_j (device)
 *   hip_stream      stream; the call synchronises it once (to check amax_x)
 *
 * Errors: MQ_ERR_INVALID_ARG (NULL or misaligned pointers, N or K <= 0, a
 * negative or non-finite amax_x value), MQ_ERR_UNSUPPORTED (N * K >= 2^31),
 * MQ_ERR_OUT_OF_MEMORY, MQ_ERR_DEVICE.
 */
mq_status mq_smooth_weights(const void* W_dev_fp16, int64_t N, int64_t K, const float* amax_x_dev_f32,
                            void* W_out_dev_fp16, int32_t* e_out_dev_i32, void* hip_stream);

/*
 * mq_smooth_activations -- X^_mj = fp16(X_mj 2^-e_j), the activations that go
 * with W^ from mq_smooth_weights (same rounding rule). X_out may be X.
 * Enqueued on hip_stream without synchronising. Errors: MQ_ERR_INVALID_ARG
 * (NULL or misaligned pointers, M or K <= 0), MQ_ERR_UNSUPPORTED
 * (M * K >= 2^31), MQ_ERR_DEVICE.
 */
mq_status mq_smooth_activations(const void* X_dev_fp16, int64_t M, int64_t K, const int32_t* e_dev_i32,
                                void* X_out_dev_fp16, void* hip_stream);

/*
 * mq_quantize_activations -- 4-bit activations for mq_linear_a4 (MosaicQuant
 * explainer, Experimental Results: weights and activations both in 4 bits;
 * Methodology section 3: quantization is a stage of the fused pipeline).
 * Each token row is quantized like the base weights, per group of G columns:
 * sx = fp16(max |x| / 7) (round half to even), qx = clamp(rne(x / sx), -7, 7),
 * qx = 0 where sx = 0; decided exactly.
 *
 *   X_dev_fp16      [M, K] fp16 activations (device, 16-byte aligned)
 *   M, K            M >= 1; K % G == 0, K <= 65536; M * Kp < 2^31 with
 *                   Kp = 128 * ceil(K / 128)
 *   group_size      G in {32, 64, 128}; must be the G of the handle the codes
 *                   are used with
 *   xq_dev_u8       [M, Kp] bytes out (device, 16-byte aligned): qx as OCP
 *                   e4m3 bytes in tile order -- for token m and column tile
 *                   kt, byte 32 g + 8 t + p of the tile's 128 bytes holds
 *                   column 128 kt + 32 t + 8 g + perm[p], perm = {0, 4, 1, 5,
 *                   2, 6, 3, 7}; columns K .. Kp - 1 hold 0
 *   xmeta_dev_u32   [M, Kp / G] out (device, 4-byte aligned): the fp16 bits of
 *                   sx in bits 0-15 and the group's code sum (int16) in bits
 *                   16-31; groups past K hold 0
 *   hip_stream      stream to enqueue on (no synchronisation)
 *
 * A group holding an inf or NaN gets a NaN scale and zero codes, so its
 * outputs in mq_linear_a4 are NaN. Errors: MQ_ERR_INVALID_ARG (NULL or
 * misaligned pointers, M or K out of range, G not supported or not dividing
 * K), MQ_ERR_UNSUPPORTED (M * Kp >= 2^31), MQ_ERR_DEVICE.
 */
mq_status mq_quantize_activations(const void* X_dev_fp16, int64_t M, int64_t K, int32_t group_size,
                                  void* xq_dev_u8, void* xmeta_dev_u32, void* hip_stream);

/*
 * mq_linear_a4 -- Y = X^ (deq(Q_base) + deq(R))^T with the 4-bit activations
 * X^ = sx * qx of mq_quantize_activations (W4A4; the residual, when the
 * handle has one, is applied inside the same kernel as in mq_linear).
 *
 *   xq_dev_u8, xmeta_dev_u32  codes and metadata from mq_quantize_activations
 *                   with this handle's K and G (device, 16- / 4-byte aligned)
 *   M               number of tokens, M >= 1; M * Kp and M * N < 2^31
 *   p               a handle from mq_pack_blocks, or from mq_pack with
 *                   residual_density giving no entries (nnz = 0)
 *   Y_dev_fp16      [M, N] fp16 output (device, 2-byte aligned, overwritten)
 *   hip_stream      stream to enqueue on (no synchronisation)
 *
 * The products run on the fp8 matrix cores exactly (4-bit integers) and each
 * group's sum is scaled and added in fp32. Up to 16 tokens one kernel runs
 * with no workspace; above that, like mq_linear's GEMM, it splits K when the
 * output tiles are few, with a stream-ordered fp32 workspace of at most
 * 16 MiB (MQ_ERR_OUT_OF_MEMORY if it cannot be had). Deterministic.
 * Errors: MQ_ERR_BAD_HANDLE, MQ_ERR_INVALID_ARG, MQ_ERR_UNSUPPORTED (a
 * handle with single residual entries: their per-entry scale cannot join the
 * integer sum; pack with mq_pack_blocks instead; or base codes of 2 GiB or
 * more), MQ_ERR_DEVICE.
 */
mq_status mq_linear_a4(const void* xq_dev_u8, const void* xmeta_dev_u32, int64_t M, const mq_packed* p,
                       void* Y_dev_fp16, void* hip_stream);

/*
 * mq_decode_a4 -- the W4A4 layer for a decode batch in one kernel: the
 * activations are quantized as mq_quantize_activations does (the same codes,
 * scales and code sums, bit for bit) inside the kernel that multiplies them,
 * so quantization runs as a stage of the fused pipeline (MosaicQuant
 * explainer, Methodology section 3) and no intermediate buffer exists.
 * Every workgroup quantizes the whole batch into its LDS, so the call is
 * limited to small batches; for more tokens use mq_quantize_activations and
 * mq_linear_a4.
 *
 *   X_dev_fp16   [M, K] fp16 activations (device, 16-byte aligned)
 *   M            1 <= M <= 2
 *   p            as for mq_linear_a4, with K <= 4096
 *   Y_dev_fp16   [M, N] fp16 output (device, 2-byte aligned, overwritten);
 *                equal, bit for bit, to mq_quantize_activations followed by
 *                mq_linear_a4 on the same X
 *   hip_stream   stream to enqueue on (no synchronisation)
 *
 * Errors: MQ_ERR_BAD_HANDLE, MQ_ERR_INVALID_ARG (NULL or misaligned
 * pointers, M <= 0), MQ_ERR_UNSUPPORTED (M > 2, K > 4096, or a handle
 * mq_linear_a4 refuses), MQ_ERR_DEVICE.
 */
mq_status mq_decode_a4(const void* X_dev_fp16, int64_t M, const mq_packed* p, void* Y_dev_fp16,
                       void* hip_stream);

/*
 * mq_stream_read -- measurement helper, not a step of the method: reads
 * `bytes` of src_dev once with 16-byte loads (workgroups of 256 threads,
 * each thread issuing all of its U = ceil(bytes / (16 * 256 * workgroups))
 * loads before using any, U <= 16) and writes the XOR of what workgroup b
 * read to sink_dev_u32[b]. Timed on a buffer of a decode layer's size, it
 * gives the streaming HBM read rate the decode kernels are compared with.
 * bytes > 0 and a multiple of 16, U <= 16, src 16-byte and sink 4-byte
 * aligned, sink holds `workgroups` words; else MQ_ERR_INVALID_ARG.
 * Enqueued only.
 */
mq_status mq_stream_read(const void* src_dev, int64_t bytes, int32_t workgroups, void* sink_dev_u32,
                         void* hip_stream);

/*
 * mq_concat -- one handle for several layers that read the same input
 * (for example the query, key and value projections, or the gate and up
 * projections of a transformer block): their rows stacked in the order
 * given, so that one mq_linear call computes all of them. This is launch
 * plumbing, not a step of the method: each part keeps the codes, scales and
 * residual selected when it was packed (its own top-k), and mq_linear on the
 * result writes Y[:, rows of part i] = mq_linear of part i, within the same
 * tolerance (the kernels may group row blocks differently).
 *
 *   parts        n handles from mq_pack (element-wise or residual-free; read
 *                only, still owned by the caller, who may free them after the
 *                call returns)
 *   n            n >= 1
 *   hip_stream   stream the copies run on; the call synchronises it
 *   out          receives the new handle (free it with mq_free)
 *
 * Every part needs the same K, group size and device, and every part but
 * the last a row count that is a multiple of 16 (whole row blocks).
 * mq_export_canonical of the result gives the parts' canonical arrays
 * concatenated row-wise (residual entries renumbered). The result owns its
 * memory: about the sum of the parts'. Errors: MQ_ERR_INVALID_ARG for a NULL
 * argument, n < 1, parts that differ in K, group size or device, or a
 * ragged part before the last; MQ_ERR_BAD_HANDLE for a handle that is not
 * live; MQ_ERR_UNSUPPORTED for a block-residual part or more than 2^31 - 1
 * weights in all; MQ_ERR_OUT_OF_MEMORY / MQ_ERR_DEVICE from HIP.
 */
mq_status mq_concat(const mq_packed* const* parts, int32_t n, void* hip_stream, mq_packed** out);

/* mq_free -- release a handle and its device memory (NULL is accepted). The
 * caller must make sure no enqueued mq_linear still reads it. */
void mq_free(mq_packed* p);

/* mq_status_string -- static, human-readable name of a status code. */
const char* mq_status_string(mq_status s);

#ifdef __cplusplus
}
#endif
#endif /* MOSAICQ_H */
