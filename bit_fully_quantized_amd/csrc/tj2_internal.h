// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tj2.h"

namespace tj2 {

// Padded storage of a quantized operand: every row holds whole 128-element
// outer blocks (nb = ceil(len/128)); the padding is written as zeros.
struct QView {
  uint8_t* codes;
  uint8_t* s16;
  float* s128;
  int64_t rows, len, nb;
  int64_t ld_codes, ld_s16, ld_s128;  // row strides in bytes, bytes, floats
  int fmt;
};

inline QView make_view(const tj2_qtensor& q) {
  QView v;
  v.codes = q.codes;
  v.s16 = q.scale16;
  v.s128 = q.scale128;
  v.rows = q.rows;
  v.len = q.len;
  v.nb = (q.len + 127) / 128;
  v.fmt = q.fmt;
  v.ld_codes = q.fmt == TJ2_NVFP4 ? v.nb * 64 : v.nb * 128;  // FP8 / NVFP6: one byte per element
  v.ld_s16 = v.nb * 8;
  v.ld_s128 = v.nb;
  return v;
}

// B operand image of a product (the f16 decode of a packed B, laid out as the
// product kernel's LDS stage): for column tile t (128 output columns) and K
// chunk g (128 elements), a block of kImgChunkBytes at (t * nchunks + g) *
// kImgChunkBytes holds row r (output column 128t + r) at r * kImgRowBytes:
// its 128 values as f16 (element k at 2k bytes), then 16 unused bytes (the
// row pitch keeps the product's fragment reads free of bank conflicts).  The
// outer scales follow the images: float S_B[g][Jpad], Jpad = 128 * tiles.
constexpr int kImgRowBytes = 272;
constexpr int kImgChunkBytes = 128 * kImgRowBytes;

struct QuantParams {
  int in_dtype;          // TJ2_BF16, TJ2_F32, TJ2_NVFP4, TJ2_FP8
  const void* x;         // dense input (BF16/F32), row-major [rows, ld_x]
  int64_t ld_x;
  QView xq;              // quantized input (NVFP4/FP8)
  int64_t rows, cols;    // logical input shape
  const int32_t* idx;    // optional column gather (row grouping)
  int64_t n_idx;
  int grouping, rounding, rht;
  uint32_t rht_mask;
  uint64_t seed, offset;
  QView out;
  // column grouping only, NVFP4 or FP8 output: also write the output's B image
  // (img != NULL): output row i is image row img_rows[i] (NULL: i), chunks of
  // img_nch, outer scales at img_sc[g * img_ld + image row]
  uint8_t* img;
  float* img_sc;
  const int32_t* img_rows;
  int64_t img_ld, img_nch;
};

hipError_t launch_quant(const QuantParams& p, hipStream_t s);

// Up to kColMultiMax column (16x1, transposed) quantizations in one launch; every
// problem shares rounding and the Hadamard switch, and is bf16 -> NVFP4,
// NVFP4 -> NVFP4 or FP8 -> FP8.
constexpr int kColMultiMax = 12;
hipError_t launch_quant_col_multi(const QuantParams* ps, int n, hipStream_t s);

// Forward split of a dense row-major input with an outlier plan: the columns
// in `rest` quantized to NVFP4 (q4) and the columns in `outl` to FP8 (q8), both
// round-to-nearest along rows, from one read of the input.
struct SplitParams {
  int in_dtype;  // TJ2_BF16 or TJ2_F32
  const void* x;
  int64_t rows, cols;
  const int32_t* rest;
  const int32_t* outl;
  QView q4, q8;
  // optional: the forward product's B image (the rows' NVFP4 chunks, then
  // their FP8 chunks from image chunk img_g8 on), written beside the codes
  uint8_t* img;
  float* img_sc;
  int64_t img_ld;  // scale row length: the rows padded to whole 128-row tiles
  int img_nch;     // chunks of the whole image
  int img_g8;
};

hipError_t launch_quant_split(const SplitParams& p, hipStream_t s);
// X (bf16) and the fp32 masters W of one forward, both split, in one launch.
hipError_t launch_quant_split2(const SplitParams& px, const SplitParams& pw, hipStream_t s);

// Both backward groupings of a bf16 [rows, cols] gradient from one read, with
// stochastic rounding: row_out [rows, cols] grouped along cols (signs row_mask,
// draws at row_offset) and col_out [cols, rows] grouped along rows (col_mask,
// col_offset); NVFP4 or NVFP6 (both outputs the same format).
struct DualParams {
  const uint16_t* x;
  int64_t rows, cols;
  QView row_out, col_out;
  uint32_t row_mask, col_mask;
  uint64_t seed, row_offset, col_offset;
  int rht;
};

hipError_t launch_quant_dual(const DualParams& p, hipStream_t s);

struct GemmSeg {
  QView a, b;  // a: [I, K], b: [J, K] grouped along K
  int64_t K;
};

struct GemmParams {
  GemmSeg seg[2];
  int nseg;
  int64_t I, J;
  void* C;
  int c_dtype;       // TJ2_F32 or TJ2_BF16
  int64_t ldc;
  const int32_t* col_map;
  int accumulate;
  float* partial;        // split-K workspace (fp32 [split][I][J]); NULL -> no split
  size_t partial_bytes;
  // outlier-column product (outl != NULL): J output columns; column outl[i]
  // (sorted, n_outl of them) takes row i of b8, the others (rest, sorted) take
  // the rows of seg[0].b in order
  QView b8;
  const int32_t* outl;
  const int32_t* rest;
  int n_outl;
  // image products: scratch for B decoded once into f16 chunk images
  // (gemm_image_bytes); NULL -> B is decoded inside the product kernel.
  // bimg_ready: the image was written by B's producer (no decode pass)
  void* bimg;
  size_t bimg_bytes;
  int bimg_ready;
};

// Number of K splits used for a product of I x J outputs over nchunks 128-element
// chunks, and the workspace it needs (0 when no split).
int gemm_split(int64_t I, int64_t J, int64_t nchunks);
size_t gemm_workspace_bytes(int64_t I, int64_t J, int64_t nchunks);

// Scratch of an image product: the f16 chunk images of a J-row B operand over
// nchunks 128-element chunks, and their outer scales.
size_t gemm_image_bytes(int64_t J, int64_t nchunks);
// Whether a product of I rows decodes its B into an image (given the room):
// only when enough row tiles would otherwise decode B again.
bool gemm_image_pays(int64_t I);
// The forward's two-segment product (NVFP4 x NVFP4, then FP8 x FP8, the first
// segment longer than one chunk) can run from a B image of both segments.
bool gemm_image_two_segments(const GemmParams& p);

hipError_t launch_gemm(const GemmParams& p, hipStream_t s);

// OsciReset and the fused master-weight pass (AdamW, then OsciReset), on up to
// kOsciMultiMax weight matrices per launch.  Parameters shared by the
// matrices of a call:
struct OsciShared {
  int mode;  // TJ2_OSCI_INIT / ACCUM / WINDOW_END (the master pass: ACCUM or WINDOW_END)
  float tau;
  int reset_enabled;
  float lr, beta1, beta2, eps, weight_decay, bc1, bc2;  // master pass only
  unsigned long long* reset_count;
  unsigned long long* flips;      // oscillation diagnostics, NULL = off
  unsigned long long* risk_hist;  // [kRiskBins], WINDOW_END only
};

// Codes written by the pass (codes == NULL: none), row strides in bytes / floats.
struct QOut {
  uint8_t* codes;
  uint8_t* s16;
  float* s128;
  int32_t ld_codes, ld_s16, ld_s128, pad;
};

inline QOut make_qout(const tj2_qtensor* q) {
  QOut o;
  o.codes = nullptr; o.s16 = nullptr; o.s128 = nullptr;
  o.ld_codes = o.ld_s16 = o.ld_s128 = o.pad = 0;
  if (!q) return o;
  const QView v = make_view(*q);
  o.codes = v.codes; o.s16 = v.s16; o.s128 = v.s128;
  o.ld_codes = (int32_t)v.ld_codes; o.ld_s16 = (int32_t)v.ld_s16; o.ld_s128 = (int32_t)v.ld_s128;
  return o;
}

// One weight matrix [N, K] and its state arrays (fp32, row-major).  With an
// outlier plan (rest != NULL) the lanes of a row cover its K1 compacted rest
// channels (NVFP4, hpr1 half groups) and then its `no` outlier channels (FP8),
// each segment padded to whole 128-element blocks; without one, K1 = K.
struct OsciProblem {
  float *W, *W_prev, *Q_prev, *dQ, *dM;  // W_prev: OsciReset only
  float *m, *v;                          // master pass only
  const float* grad;                     // master pass only
  int32_t N, K;
  const int32_t* rest;
  const int32_t* outl;
  int32_t K1, no;
  int32_t hpr, hpr1;  // half groups (8 elements) per row: all segments, the rest segment
  QOut wq, w8;        // forward codes of the final W: NVFP4 [N, K1], FP8 [N, no]
};

constexpr int kRiskBins = 32;
constexpr int kOsciMultiMax = 16;

struct OsciLaunch {
  OsciShared c;
  OsciProblem p[kOsciMultiMax];
  uint32_t begin[kOsciMultiMax + 1];
  int n;
};
static_assert(sizeof(OsciLaunch) <= 4096, "kernel arguments stay within 4 KB");

hipError_t launch_osci_multi(const OsciShared& c, const OsciProblem* ps, int n, bool master, hipStream_t s);

// Calibration sums: rows per slab of the first pass; the second pass adds the
// slabs' fp64 partial sums (workspace [ceil(M / kSumsqRows)][K]) in slab order.
constexpr int kSumsqRows = 512;
size_t sumsq_workspace_bytes(int64_t M, int64_t K);
hipError_t launch_channel_sumsq(const void* X, int64_t M, int64_t K, double* acc, double* partial, hipStream_t s);

}  // namespace tj2
