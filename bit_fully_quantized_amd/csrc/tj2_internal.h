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
};

hipError_t launch_quant_split(const SplitParams& p, hipStream_t s);

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
};

// Number of K splits used for a product of I x J outputs over nchunks 128-element
// chunks, and the workspace it needs (0 when no split).
int gemm_split(int64_t I, int64_t J, int64_t nchunks);
size_t gemm_workspace_bytes(int64_t I, int64_t J, int64_t nchunks);

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
