/*
 * tj2.h -- C ABI of libtj2: the TetraJet-v2 NVFP4 double-block quantized linear
 * layer, OsciReset and OutControl outlier channels on AMD Instinct MI355X (gfx950).
 *
 * Method source: "TetraJet-v2: Accurate NVFP4 Training for Large Language Models
 * with Oscillation Suppression and Outlier Control" as summarised on the
 * gist.science technical-summary pages (sections cited per entry point below).
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library never
 *    allocates device memory.  Host-side descriptors (tj2_qtensor, tj2_outlier_plan,
 *    the tj2_osci_tensor / tj2_master_tensor arrays of the _multi entry points)
 *    are read during the call only.
 *  - Dense tensors are row-major and contiguous.  bf16 is passed as raw 16-bit
 *    words.  Device pointers must be 16-byte aligned.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream).  Calls return once the work is enqueued.
 *  - Return value: TJ2_OK, or an error code with a message in tj2_last_error()
 *    (thread-local).  Argument checks happen before any launch, so an error
 *    other than TJ2_ERR_HIP means nothing was enqueued.
 *  - Data-dependent conditions (NaN/Inf inputs) are not checked; results for
 *    them are unspecified.
 *  - Calls that share output buffers must be ordered by the caller (streams).
 */
#ifndef TJ2_H_
#define TJ2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tj2_status;
#define TJ2_OK 0
#define TJ2_ERR_ARG 1         /* null pointer, bad enum, out-of-range value     */
#define TJ2_ERR_SHAPE 2       /* dimension not a multiple of 16, mismatch        */
#define TJ2_ERR_ALIGN 3       /* device pointer not 16-byte aligned              */
#define TJ2_ERR_HIP 4         /* launch or runtime error reported by HIP         */
#define TJ2_ERR_UNSUPPORTED 5 /* valid but unimplemented combination             */

/* element / storage types */
#define TJ2_BF16 0
#define TJ2_F32 1
#define TJ2_NVFP4 2
#define TJ2_FP8 3
#define TJ2_NVFP6 4 /* E2M3 elements in the NVFP4 double block (the FP6 x FP4 variant) */

/* grouping of a quantizer */
#define TJ2_GROUP_ROW 0 /* 1x16 groups along the contiguous (column) dimension   */
#define TJ2_GROUP_COL 1 /* 16x1 groups along rows; the output is stored transposed */

/* element rounding */
#define TJ2_RTN 0 /* round to nearest, ties to even (forward pass)            */
#define TJ2_SR 1  /* stochastic rounding with Philox4x32-10 draws (backward)  */

/* OsciReset modes */
#define TJ2_OSCI_INIT 0
#define TJ2_OSCI_ACCUM 1
#define TJ2_OSCI_WINDOW_END 2

/*
 * A quantized operand with `rows` rows of `len` elements, grouped along `len`
 * (TetraJet-v2 technical summary, section 2.A: 16-element inner blocks with an
 * 8-bit scale, 128-element outer blocks with an FP32 scale).
 *
 * Storage, with nb = ceil(len / 128):
 *   TJ2_NVFP4: codes    uint8 [rows][nb*64]  E2M1, element 2i in the low nibble of byte i
 *              scale16  uint8 [rows][nb*8]   E4M3FN, one per 16 elements
 *              scale128 float [rows][nb]     one per 128 elements
 *   TJ2_FP8:   codes    uint8 [rows][nb*128] E4M3FN
 *              scale16  unused (may be NULL)
 *              scale128 float [rows][nb]
 *   TJ2_NVFP6: codes    uint8 [rows][nb*128] E2M3 values, each stored as the
 *                                            E4M3FN byte of that value
 *              scale16  uint8 [rows][nb*8]   E4M3FN, one per 16 elements
 *              scale128 float [rows][nb]     one per 128 elements (amax / 3360)
 * Element positions beyond `len` in each row are padding; producers write
 * them as zero.  `len` must be a positive multiple of 16.
 * E2M1 code: bit 3 sign, bits 2..0 index into {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 */
typedef struct {
  uint8_t* codes;
  uint8_t* scale16;
  float* scale128;
  int64_t rows;
  int64_t len;
  int32_t fmt;
  int32_t reserved;
} tj2_qtensor;

/*
 * Static outlier channels (OutControl; technical summary, section 2.C): the
 * input channels kept in FP8 and the complement kept in NVFP4.  Both are
 * DEVICE int32 arrays in ascending order that together list every channel
 * 0..K-1 once.  n_outliers must be a positive multiple of 16.
 */
typedef struct {
  const int32_t* outliers;
  const int32_t* rest;
  int32_t n_outliers;
  int32_t reserved;
} tj2_outlier_plan;

/*
 * Buffers for the backward operands (optional argument of nvfp4_linear_bwd).
 * w_given != 0: Wt (and W8t with a plan) already hold this call's re-grouped
 * weight operands (the dX mask, SR at offset + 1 / offset + 4), e.g. written
 * by master_update_step's `next` output, and the call reads them instead of
 * forming them from Wq / W8.
 */
typedef struct {
  tj2_qtensor dYq;  /* [M, N] NVFP4, groups along N (RHT_N, SR)       */
  tj2_qtensor dYt;  /* [N, M] NVFP4, groups along M (RHT_M, SR)       */
  tj2_qtensor Wt;   /* [K1, N] NVFP4, re-grouped dequantized weights  */
  tj2_qtensor Xt;   /* [K1, M] NVFP4, re-grouped dequantized inputs   */
  tj2_qtensor W8t;  /* [n_outliers, N] FP8 (plan only)                */
  tj2_qtensor X8t;  /* [n_outliers, M] FP8 (plan only)                */
  int32_t w_given;
  int32_t reserved;
} tj2_bwd_operands;

/* Message describing the last error of the calling thread ("" if none). */
const char* tj2_last_error(void);

/* Library version string. */
const char* tj2_version(void);

/*
 * Bytes needed by each array of a tj2_qtensor of the given format and shape
 * (see the storage table above).  Host-only; returns TJ2_ERR_ARG / _SHAPE for
 * a bad format or a len that is not a positive multiple of 16.
 */
tj2_status tj2_qtensor_bytes(int32_t fmt, int64_t rows, int64_t len, size_t* codes_bytes,
                             size_t* scale16_bytes, size_t* scale128_bytes);

/*
 * 16-bit sign mask of the random Hadamard transform for one product (bit j set
 * = position j of every 16-chunk is negated).  Host function, no device work:
 * low 16 bits of word 0 of Philox4x32-10 with key (lo seed, hi seed) and counter
 * (0xFFFFFFFF, 0xFFFFFFFF, lo offset, hi offset).  (Section 2.C: RHT on dX, dW.)
 * Entry points that take a mask take it as uint32_t and use its low 16 bits.
 */
uint16_t tj2_rht_signs(uint64_t seed, uint64_t offset);

/*
 * Double-block quantizer (section 2.A; FP8 output for the OutControl channels,
 * section 2.C).
 *
 * Input: a logical [rows, cols] tensor, either dense (x_dtype TJ2_BF16 / TJ2_F32,
 * `x` points to rows*cols elements, x_q ignored) or quantized (x_dtype TJ2_NVFP4
 * / TJ2_FP8, `x` ignored, *x_q describes rows x cols grouped along cols), in
 * which case it is dequantized first ((q*s)*S, or e*S8, in fp32).
 *
 * col_idx (optional, device int32[n_idx], TJ2_GROUP_ROW with dense input only):
 * quantize the gathered columns x[:, col_idx] instead of all columns.
 *
 * grouping TJ2_GROUP_ROW: groups along cols; *out is [rows, n] with n = n_idx or cols.
 * grouping TJ2_GROUP_COL: groups along rows (16x1); *out is [cols, rows] (transposed).
 * The grouped length must be a multiple of 16; for TJ2_GROUP_COL, cols too.
 *
 * rht != 0: apply the 16-wide Hadamard transform with sign mask rht_signs along
 * the grouping dimension before quantizing.
 * rounding TJ2_SR: element e (row-major index in the output, i.e. in the grouped
 * layout: for TJ2_GROUP_COL, output row = input column) draws 16 bits from
 * Philox4x32-10 block e>>3 (counter (lo, hi of e>>3, lo, hi of offset), key seed),
 * word (e>>1)&3, half e&1 (0 = low half).
 *
 * out->fmt selects NVFP4 (scale = amax/2688 per 128, E4M3 round-up per 16), FP8
 * (E4M3FN elements, scale = amax/448 per 128) or NVFP6 (E2M3 elements, largest
 * 7.5, scale = amax/3360 per 128, E4M3 round-up per 16; dense input only; the
 * FP6 operand of the FP6 x FP4 variant the pages name as future work, section
 * 5).  out->rows/len must match.
 */
tj2_status nvfp4_quantize(const void* x, int32_t x_dtype, const tj2_qtensor* x_q, int64_t rows,
                          int64_t cols, const int32_t* col_idx, int64_t n_idx, int32_t grouping,
                          int32_t rounding, int32_t rht, uint32_t rht_signs, uint64_t seed,
                          uint64_t offset, tj2_qtensor* out, void* stream);

/*
 * The output gradient's two backward operands from one read (section 2.A: dY
 * enters dX grouped along N and dW grouped along M; section 2.C: each with a
 * 16-wide random Hadamard transform): x bf16 [rows, cols] row-major (16-byte
 * aligned, rows and cols multiples of 16) -> row_out [rows, cols] grouped along cols
 * (Hadamard signs tj2_rht_signs(seed, row_offset), stochastic draws at
 * row_offset) and col_out [cols, rows] grouped along rows, stored transposed
 * (signs tj2_rht_signs(seed, col_offset), draws at col_offset).  Both outputs
 * TJ2_NVFP4, or both TJ2_NVFP6; rht = 0 skips the transforms.  The codes,
 * scales and draws equal those of two nvfp4_quantize calls (TJ2_SR, the same
 * signs and offsets); nvfp4_linear_bwd quantizes dY with it (row_offset =
 * offset, col_offset = offset + 2).
 */
tj2_status nvfp4_quantize_dual(const void* x, int64_t rows, int64_t cols, int32_t rht, uint64_t seed,
                               uint64_t row_offset, uint64_t col_offset, tj2_qtensor* row_out,
                               tj2_qtensor* col_out, void* stream);

/*
 * Product on packed operands (section 2: every linear-layer product runs on the
 * quantized tensors).  C[i, col(j)] (+)= sum_k A[i,k] B[j,k] + sum_k A2[i,k] B2[j,k]
 * with A [I, K] and B [J, K] grouped along K, each NVFP4 or FP8; the optional
 * second segment (A2, B2: [I, K2], [J, K2]) adds another reduction range.
 * The result is accumulated in fp32 with one FP32 promotion per 128-element
 * outer block.  c_dtype TJ2_F32 or TJ2_BF16 (round to nearest even); ldc in
 * elements.  col_map (optional, device int32[J]) gives the output column of B
 * row j.  accumulate != 0 adds into C (TJ2_F32 only).
 * workspace: fp32 partial sums of a K split (the library splits K only when
 * the output has too few 256x128 tiles to fill the GPU), then, for a product
 * of at least 2048 rows (one segment, or an NVFP4 segment of more than 128
 * followed by an FP8 one when the product runs without a split), room for B
 * decoded once into an f16 image that the product copies into LDS instead of
 * decoding B again in every row tile (a second segment's chunks follow the
 * first's): nvfp4_gemm_workspace_size(I, J, A->len, A2 ? A2->len : 0)
 * bytes for both (0 when neither applies).  NULL runs the product without a
 * split or an image; a non-NULL workspace smaller than the partial sums need is
 * an error (TJ2_ERR_ARG); one that holds the partial sums but not the image
 * runs without the image.  The results do not depend on the image (the same
 * f16 values, the same order of operations).
 */
tj2_status nvfp4_gemm(const tj2_qtensor* A, const tj2_qtensor* B, const tj2_qtensor* A2,
                      const tj2_qtensor* B2, void* C, int32_t c_dtype, int64_t ldc,
                      const int32_t* col_map, int32_t accumulate, void* workspace, size_t ws_bytes,
                      void* stream);
/* Workspace of nvfp4_gemm for I x J outputs over reductions of K (and K2 for a
 * second segment, else 0) elements, image included; the same for
 * nvfp4_gemm_outlier_cols with K2 = 0.  Returns 0 for invalid sizes. */
size_t nvfp4_gemm_workspace_size(int64_t I, int64_t J, int64_t K, int64_t K2);

/*
 * nvfp4_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, kernels and results as nvfp4_gemm with a workspace of
 * nvfp4_gemm_workspace_size(...) bytes, but the split-K partial sums live in a
 * static device array of the library (32 MiB, one per GPU, held until the
 * process ends), so the call allocates nothing.  A product whose K split needs
 * more than 32 MiB of partial sums is refused with TJ2_ERR_SHAPE before any
 * work (the 370M-style weight gradients need at most 32 MiB).  The array's
 * device address is looked up on the first call on each device (the current
 * device must be the stream's).  Every call on one GPU shares that array:
 * calls that overlap on one GPU (different streams, or host threads) race and
 * must be ordered by the caller.  Nothing in the array needs clearing: each
 * split writes every partial sum before the reduction reads it.
 */
tj2_status nvfp4_gemm_noalloc(const tj2_qtensor* A, const tj2_qtensor* B, const tj2_qtensor* A2,
                              const tj2_qtensor* B2, void* C, int32_t c_dtype, int64_t ldc,
                              const int32_t* col_map, int32_t accumulate, void* stream);

/*
 * Product whose output columns are split by a static outlier plan (OutControl,
 * TetraJet-v2 technical summary, section 2.C), in one launch: with
 * J = B->rows + B8->rows output columns,
 *   C[i, plan->rest[j]]     = sum_k A[i,k] B[j,k]    (B NVFP4, j < B->rows)
 *   C[i, plan->outliers[j]] = sum_k A[i,k] B8[j,k]   (B8 FP8, j < n_outliers)
 * This is how the backward forms dX (B = re-grouped W-hat of the non-outlier
 * channels, B8 = its FP8 outlier channels) and dW (B, B8 = re-grouped X-hat).
 * A [I, K] NVFP4 (or NVFP6); B [J - n, K] NVFP4; B8 [n, K] FP8 with n = plan->n_outliers;
 * plan arrays sorted ascending, device int32, 16-byte aligned, rest listing the
 * J - n columns not in outliers.  C, ldc (>= J), c_dtype, accumulate and the
 * workspace (nvfp4_gemm_workspace_size(I, J, K, 0) bytes) as for nvfp4_gemm.
 */
tj2_status nvfp4_gemm_outlier_cols(const tj2_qtensor* A, const tj2_qtensor* B, const tj2_qtensor* B8,
                                   const tj2_outlier_plan* plan, void* C, int32_t c_dtype, int64_t ldc,
                                   int32_t accumulate, void* workspace, size_t ws_bytes, void* stream);

/*
 * Forward of the NVFP4 linear layer Y = X W^T (section 2.A), X [M, K] bf16,
 * W [N, K].
 *   W_master != NULL: quantize the fp32 masters into *Wq (and *W8 with a plan);
 *   W_master == NULL: use *Wq (*W8) as given (e.g. codes emitted by osci_reset_step).
 *   plan == NULL: Xq [M, K], Wq [N, K] NVFP4 (RTN, 1x16 along K); X8/W8 unused.
 *   plan != NULL: Xq [M, K1], Wq [N, K1] hold the compacted non-outlier channels
 *     (K1 = K - n_outliers) in NVFP4; X8 [M, n_outliers], W8 [N, n_outliers] the
 *     outlier channels in FP8 (round to nearest even); Y adds both products.
 * Xq/X8 are saved for the backward and stay owned by the caller.
 * Y [M, N]: y_dtype TJ2_BF16 or TJ2_F32.  M, K, N multiples of 16.
 * workspace: split-K partial sums of the product (few output tiles, e.g. a
 * small M), then, with a plan, room for the product's B image (W-hat's NVFP4
 * chunks then W8's FP8 chunks, decoded to f16, 2.125 B per weight), which the
 * split quantization of W_master writes beside Wq and W8 when M >= 2048, K <=
 * 8192, K - n_outliers > 128 and the product runs unsplit;
 * nvfp4_linear_fwd_workspace_size(M, N, K, n_outliers) bytes covers both.
 * NULL runs the product unsplit and without the image; a workspace smaller
 * than the partial sums is TJ2_ERR_ARG, one without room for the image runs the
 * product without it (same result, bit for bit).
 */
tj2_status nvfp4_linear_fwd(const void* X, int64_t M, int64_t K, int64_t N, const float* W_master,
                            tj2_qtensor* Wq, tj2_qtensor* W8, const tj2_outlier_plan* plan,
                            tj2_qtensor* Xq, tj2_qtensor* X8, void* Y, int32_t y_dtype,
                            void* workspace, size_t ws_bytes, void* stream);
size_t nvfp4_linear_fwd_workspace_size(int64_t M, int64_t N, int64_t K, int32_t n_outliers);

/*
 * Backward of the NVFP4 linear layer (sections 2.A and 2.C).  Uses the forward's
 * quantized tensors (X-hat / W-hat alignment), a 16-wide random Hadamard
 * transform along the reduction dimension of each product (signs
 * tj2_rht_signs(seed, offset+0) for dX, (seed, offset+2) for dW; rht == 0 skips
 * it) and stochastic rounding with Philox offsets
 *   offset+0 dY (groups along N), offset+1 W-hat re-grouped along N,
 *   offset+2 dY re-grouped along M, offset+3 X-hat re-grouped along M,
 *   offset+4 FP8 W-hat outliers, offset+5 FP8 X-hat outliers.
 * The caller advances offset by 8 per call.
 *   dX [M, K] (dx_dtype TJ2_BF16 or TJ2_F32) = Q(dY T) . Q(T^T W-hat)
 *   dW [N, K] fp32                           = Q(dY^T T) . Q(T^T X-hat)
 * With a plan, outlier columns of dX / dW come from the FP8 operands and are
 * scattered back to their original channel positions.
 * ops (optional): caller buffers for the intermediate operands (shapes in
 * tj2_bwd_operands); NULL = carve them from `workspace`, which must then hold
 * nvfp4_linear_bwd_workspace_size(M, N, K, n_outliers) bytes.  That size also
 * covers the split-K partial sums and the B images of the two products (dX for
 * M >= 2048, dW for N >= 2048), which the column re-grouping of W-hat and
 * X-hat writes as it quantizes; with ops given, a workspace that holds them
 * (NULL or smaller: products without them) is used the same way.
 */
tj2_status nvfp4_linear_bwd(const void* dY, int64_t M, int64_t N, int64_t K, const tj2_qtensor* Xq,
                            const tj2_qtensor* X8, const tj2_qtensor* Wq, const tj2_qtensor* W8,
                            const tj2_outlier_plan* plan, int32_t rht, uint64_t seed,
                            uint64_t offset, void* dX, int32_t dx_dtype, float* dW,
                            tj2_bwd_operands* ops, void* workspace, size_t ws_bytes, void* stream);
size_t nvfp4_linear_bwd_workspace_size(int64_t M, int64_t N, int64_t K, int32_t n_outliers);

/*
 * The FP6 x FP4 backward (technical summary, section 5 names FP6 x FP4 mixed
 * precision as a future direction; reading: the gradient operand takes the
 * wider element): nvfp4_linear_bwd with the two dY operands (ops->dYq [M, N],
 * ops->dYt [N, M]) in TJ2_NVFP6 -- E2M3 elements under the same E4M3 inner and
 * FP32 outer scales, the same Hadamard masks, Philox offsets and stochastic
 * rounding rule -- while the re-grouped W-hat and X-hat stay NVFP4 (and FP8
 * under a plan).  Arguments, outputs and errors as for nvfp4_linear_bwd; the
 * workspace (ops == NULL) holds nvfp6x4_linear_bwd_workspace_size(M, N, K,
 * n_outliers) bytes.
 */
tj2_status nvfp6x4_linear_bwd(const void* dY, int64_t M, int64_t N, int64_t K, const tj2_qtensor* Xq,
                              const tj2_qtensor* X8, const tj2_qtensor* Wq, const tj2_qtensor* W8,
                              const tj2_outlier_plan* plan, int32_t rht, uint64_t seed, uint64_t offset,
                              void* dX, int32_t dx_dtype, float* dW, tj2_bwd_operands* ops, void* workspace,
                              size_t ws_bytes, void* stream);
size_t nvfp6x4_linear_bwd_workspace_size(int64_t M, int64_t N, int64_t K, int32_t n_outliers);

/*
 * Oscillation diagnostics (optional in osci_reset_step and master_update_step).
 * Section 1 of the TetraJet-v2 technical summary names the failure mode they
 * measure: small master updates that flip the quantized weight back and forth
 * between adjacent bins; section 2.B defines the risk dist_Q / dist_M.  Both
 * members are device uint64 counters that the call adds to (the caller zeroes
 * them, e.g. at a window start); NULL members are skipped, as is a NULL diag.
 *   flips:     ACCUM / WINDOW_END: the number of elements whose E2M1 code (bin
 *              and sign) in the forward quantization of W differs from that of
 *              the previous master (W_prev; for master_update_step the master
 *              before the update), before any reset; +0 and -0 are one bin.
 *              Codes are compared, not Q values: a block's FP32 scale moves with
 *              its largest element, which changes Q without a change of bin.
 *   risk_hist: [TJ2_RISK_BINS], WINDOW_END only: each element's window risk,
 *              with dQ and dM as accumulated up to this step (before the reset
 *              decision and the zeroing): bin 0 if dQ == 0; bin 31 if dQ > 0 and
 *              dM == 0; otherwise, with r = dQ / dM rounded to fp32 and e its
 *              binary exponent (floor(log2 r)), bin min(max(e + 16, 1), 30).
 * Both pointers must be 8-byte aligned (TJ2_ERR_ALIGN).
 */
#define TJ2_RISK_BINS 32
typedef struct {
  uint64_t* flips;
  uint64_t* risk_hist;
} tj2_osci_diag;

/*
 * OsciReset (section 2.B) on fp32 masters W [N, K] and its state arrays (all
 * fp32 [N, K], caller-owned).  Q(w) is the forward quantizer dequantized in
 * fp32: RTN NVFP4 in 1x16 groups along K; with an outlier plan (section 2.C)
 * NVFP4 over the compacted rest channels and FP8 (E4M3, per-128 FP32 scale,
 * round to nearest even) over the outlier channels, as nvfp4_linear_fwd
 * quantizes the masters, so an outlier weight is reset to its FP8 point.
 *   TJ2_OSCI_INIT:       W_prev = W, Q_prev = Q(W), dQ = dM = 0.
 *   TJ2_OSCI_ACCUM:      dQ += |Q(W) - Q_prev|, dM += |W - W_prev|, Q_prev = Q(W), W_prev = W.
 *   TJ2_OSCI_WINDOW_END: as ACCUM; then where reset_enabled and dQ > tau*dM:
 *                        W = Q(W), W_prev = Q(W); then dQ = dM = 0.
 * plan (optional): device index lists as for nvfp4_linear_fwd.  With a plan,
 * the state arrays W_prev, Q_prev, dQ, dM hold each row in the plan's
 * compacted channel order (position p < K1 is channel rest[p], position
 * K1 + i is channel outliers[i]), so the pass reads them contiguously; W
 * stays in channel order.  A plan must be the same from INIT on.
 * Wq_out (optional, NVFP4 [N, K1], K1 = K - n_outliers): forward codes of the
 * final W; W8_out (optional, plan only, FP8 [N, n_outliers]): its FP8 codes.
 * Together they are the forward's weight operands (nvfp4_linear_fwd with
 * W_master == NULL).
 * reset_count (optional, device uint64): incremented by the number of resets.
 * diag (optional): oscillation diagnostics (tj2_osci_diag; a flip of an
 * outlier weight is a change of its E4M3 code).
 * K must be a multiple of 16.
 * The pages give the risk threshold and the window as parameters without
 * values: tau is an argument and the window is the caller's count of calls
 * between TJ2_OSCI_INIT / TJ2_OSCI_WINDOW_END.
 */
tj2_status osci_reset_step(float* W, float* W_prev, float* Q_prev, float* dQ, float* dM, int64_t N,
                           int64_t K, int32_t mode, float tau, int32_t reset_enabled,
                           const tj2_outlier_plan* plan, tj2_qtensor* Wq_out, tj2_qtensor* W8_out,
                           uint64_t* reset_count, const tj2_osci_diag* diag, void* stream);

/*
 * One OsciReset problem of osci_reset_step_multi: W [N, K], its state arrays
 * (all fp32 [N, K], caller-owned device memory), an optional plan and optional
 * codes Wq_out / W8_out (host descriptors), as for osci_reset_step.
 */
typedef struct {
  float* W;
  float* W_prev;
  float* Q_prev;
  float* dQ;
  float* dM;
  int64_t N;
  int64_t K;
  tj2_qtensor* Wq_out;
  const tj2_outlier_plan* plan;
  tj2_qtensor* W8_out;
} tj2_osci_tensor;

/*
 * osci_reset_step (section 2.B) on n independent weight matrices with one mode,
 * tau, reset switch and set of counters, in as few launches as possible (up to
 * 16 matrices per launch) instead of one per matrix: the step that follows an
 * optimizer update of a whole model.  Results equal n osci_reset_step calls.
 * `tensors` is a host array of n (>= 1) descriptors, read during the call;
 * every member is checked as in osci_reset_step before anything is enqueued.
 * reset_count and diag accumulate over all matrices.
 */
tj2_status osci_reset_step_multi(const tj2_osci_tensor* tensors, int32_t n, int32_t mode, float tau,
                                 int32_t reset_enabled, uint64_t* reset_count, const tj2_osci_diag* diag,
                                 void* stream);

/*
 * AdamW hyper-parameters of one optimizer step on the fp32 masters (the pages
 * train with fp32 masters but do not name the optimizer; AdamW with decoupled
 * weight decay is this library's choice).  bias_correction1 = 1 - beta1^t and
 * bias_correction2 = 1 - beta2^t for step t >= 1, computed by the caller.
 */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay, bias_correction1, bias_correction2;
} tj2_adamw_params;

/*
 * The next backward's weight operands, formed by the master pass from the codes
 * it writes (section 2.A: the backward re-groups the forward's quantized
 * weights W-hat in 16x1 groups along N): Wt [K1, N] NVFP4 = SR of the
 * Hadamard-transformed W-hat along N at offset + 1, W8t [n_outliers, N] FP8
 * (plan only) at offset + 4, both with the dX mask tj2_rht_signs(seed,
 * offset + 0) (rht == 0: no transform) -- bit for bit what nvfp4_linear_bwd
 * with this seed and offset forms from the same Wq / W8.  Pass them to that
 * call with tj2_bwd_operands.w_given.  Host descriptor, read during the call.
 */
typedef struct {
  tj2_qtensor* Wt;
  tj2_qtensor* W8t;
  uint64_t seed;
  uint64_t offset;
  int32_t rht;
  int32_t reserved;
} tj2_next_bwd;

/*
 * Fused master-weight pass: one AdamW step on the fp32 masters W [N, K], then
 * OsciReset (section 2.B) of the updated masters, then their forward codes, in
 * one pass over W, the moments m, v, the gradient grad and the OsciReset state
 * Q_prev, dQ, dM (all fp32 [N, K], caller-owned, updated in place except grad).
 * Per element, fp32, each operation rounded to nearest (no fused multiply-add):
 *   m' = beta1*m + (1-beta1)*g;  v' = beta2*v + (1-beta2)*(g*g)
 *   u  = (m'/bc1) / (sqrt(v'/bc2) + eps)
 *   W' = W*(1 - lr*wd) - lr*u
 *   then OsciReset on W' with W_prev = W (the pre-update master, so no W_prev
 *   array): mode TJ2_OSCI_ACCUM or TJ2_OSCI_WINDOW_END as in osci_reset_step
 *   (TJ2_OSCI_INIT is osci_reset_step's; its W_prev is not read here).
 * plan, Wq_out, W8_out, reset_count, diag: as in osci_reset_step; with a plan
 * the moments m, v are kept in the compacted channel order as well (W and
 * grad stay in channel order).
 * next (optional): also form the next backward's weight operands from the
 * written codes (needs Wq_out, and W8_out with a plan; N a multiple of 16).
 * K must be a multiple of 16; arrays 16-byte aligned.  Errors: TJ2_ERR_ARG
 * (NULL array or params, bad mode, tau < 0), TJ2_ERR_SHAPE, TJ2_ERR_ALIGN.
 */
tj2_status master_update_step(float* W, float* m, float* v, const float* grad, float* Q_prev, float* dQ,
                              float* dM, int64_t N, int64_t K, const tj2_adamw_params* adam, int32_t mode,
                              float tau, int32_t reset_enabled, const tj2_outlier_plan* plan,
                              tj2_qtensor* Wq_out, tj2_qtensor* W8_out, const tj2_next_bwd* next,
                              uint64_t* reset_count, const tj2_osci_diag* diag, void* stream);

/*
 * One weight matrix of master_update_step_multi: the masters W [N, K], moments
 * m, v, gradient grad and OsciReset state Q_prev, dQ, dM (all fp32 [N, K],
 * caller-owned device memory), and the optional plan, codes and next-backward
 * operands of master_update_step (host descriptors).
 */
typedef struct {
  float* W;
  float* m;
  float* v;
  const float* grad;
  float* Q_prev;
  float* dQ;
  float* dM;
  int64_t N;
  int64_t K;
  tj2_qtensor* Wq_out;
  const tj2_outlier_plan* plan;
  tj2_qtensor* W8_out;
  const tj2_next_bwd* next;
} tj2_master_tensor;

/*
 * master_update_step on n weight matrices with one set of AdamW parameters,
 * mode, tau, reset switch and counters, up to 16 matrices per launch (the
 * optimizer step of a whole model).  Results equal n master_update_step calls.
 * `tensors` is a host array of n (>= 1) descriptors, read during the call;
 * every member is checked as in master_update_step before anything is
 * enqueued (the error names the first bad index).  reset_count and diag
 * accumulate over all matrices.
 */
tj2_status master_update_step_multi(const tj2_master_tensor* tensors, int32_t n, const tj2_adamw_params* adam,
                                    int32_t mode, float tau, int32_t reset_enabled, uint64_t* reset_count,
                                    const tj2_osci_diag* diag, void* stream);

/*
 * OutControl calibration (technical summary, section 2.C: the top p% channels
 * are chosen once from a short calibration window and stay in FP8).
 *
 * tj2_channel_sumsq: acc[k] += sum over rows m of X[m, k]^2 for a bf16 X [M, K]
 * (device), acc a device fp64 [K] array that the caller zeroes once and passes
 * for every calibration batch.  Squares and sums are fp64 in a fixed order
 * (per 512-row slab, then slab by slab), so a result does not depend on
 * scheduling.  workspace: device, tj2_channel_sumsq_workspace_size(M, K)
 * bytes, 16-byte aligned.  K a multiple of 16.
 */
size_t tj2_channel_sumsq_workspace_size(int64_t M, int64_t K);
tj2_status tj2_channel_sumsq(const void* X, int64_t M, int64_t K, double* acc, void* workspace, size_t ws_bytes,
                             void* stream);

/*
 * tj2_select_outliers: the static plan from the channel scores (host function,
 * no device work).  n = ceil(p * K / 16) * 16 channels with the largest scores
 * (ties to the lower channel index) are the outliers; every other channel is
 * in rest.  scores: host double [K] (non-negative, finite); outliers: host
 * int32 [n] and rest: host int32 [K - n], both written in ascending order
 * (size them for p, e.g. K entries each); *n_outliers receives n.  The caller
 * copies both lists to the device for a tj2_outlier_plan.  Errors: TJ2_ERR_ARG
 * (NULL pointer, p outside (0, 1), a negative or non-finite score),
 * TJ2_ERR_SHAPE (K not a positive multiple of 16, or n >= K).
 */
tj2_status tj2_select_outliers(const double* scores, int64_t K, double p, int32_t* outliers, int32_t* rest,
                               int32_t* n_outliers);

#ifdef __cplusplus
}
#endif
#endif /* TJ2_H_ */
