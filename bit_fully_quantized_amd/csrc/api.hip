// C ABI of libtj2 (declared in include/tj2.h): argument validation and the
// orchestration of the linear layer's forward and backward passes over the
// quantizer, product and OsciReset kernels.  All device work is enqueued on
// the caller's stream; no device memory is allocated here.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "tj2_internal.h"

using namespace tj2;

namespace {

thread_local std::string g_err;

tj2_status fail(tj2_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tj2_status fail(tj2_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

tj2_status ok() {
  g_err.clear();
  return TJ2_OK;
}

tj2_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TJ2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return TJ2_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define TJ2_TRY(expr)                 \
  do {                                \
    tj2_status st_ = (expr);          \
    if (st_ != TJ2_OK) return st_;    \
  } while (0)

tj2_status check_qtensor(const tj2_qtensor* q, const char* name, int fmt, int64_t rows, int64_t len) {
  if (!q) return fail(TJ2_ERR_ARG, "%s is NULL", name);
  if (q->fmt != fmt) return fail(TJ2_ERR_ARG, "%s has format %d, expected %d", name, q->fmt, fmt);
  if (q->rows != rows || q->len != len)
    return fail(TJ2_ERR_SHAPE, "%s is [%lld, %lld], expected [%lld, %lld]", name, (long long)q->rows,
                (long long)q->len, (long long)rows, (long long)len);
  if (len <= 0 || len % 16) return fail(TJ2_ERR_SHAPE, "%s: len %lld is not a positive multiple of 16", name, (long long)len);
  if (rows <= 0) return fail(TJ2_ERR_SHAPE, "%s: rows must be positive", name);
  // the products index 128-element blocks (row * blocks per row) in 32 bits
  if (rows * ((len + 127) / 128) >= ((int64_t)1 << 32)) return fail(TJ2_ERR_SHAPE, "%s: too many 128-element blocks", name);
  if (fmt != TJ2_NVFP4 && fmt != TJ2_FP8 && fmt != TJ2_NVFP6) return fail(TJ2_ERR_ARG, "%s: bad format %d", name, fmt);
  const bool has_s16 = fmt != TJ2_FP8;
  if (!q->codes || !q->scale128 || (has_s16 && !q->scale16))
    return fail(TJ2_ERR_ARG, "%s: NULL array", name);
  if (!aligned16(q->codes) || !aligned16(q->scale128) || (has_s16 && !aligned16(q->scale16)))
    return fail(TJ2_ERR_ALIGN, "%s: arrays must be 16-byte aligned", name);
  return TJ2_OK;
}

// Device counters of the oscillation diagnostics (NULL diag or members: off).
tj2_status diag_pointers(const tj2_osci_diag* d, unsigned long long** flips, unsigned long long** hist) {
  *flips = nullptr;
  *hist = nullptr;
  if (!d) return TJ2_OK;
  if ((reinterpret_cast<uintptr_t>(d->flips) & 7u) || (reinterpret_cast<uintptr_t>(d->risk_hist) & 7u))
    return fail(TJ2_ERR_ALIGN, "diagnostic counters must be 8-byte aligned");
  *flips = reinterpret_cast<unsigned long long*>(d->flips);
  *hist = reinterpret_cast<unsigned long long*>(d->risk_hist);
  return TJ2_OK;
}

tj2_status check_dims(int64_t v, const char* name) {
  if (v <= 0 || v % 16) return fail(TJ2_ERR_SHAPE, "%s = %lld must be a positive multiple of 16", name, (long long)v);
  if (v > (int64_t)1 << 30) return fail(TJ2_ERR_SHAPE, "%s = %lld is too large", name, (long long)v);
  return TJ2_OK;
}

size_t qbytes(int fmt, int64_t rows, int64_t len, size_t* c, size_t* s16, size_t* s128) {
  const int64_t nb = (len + 127) / 128;
  *c = (size_t)(rows * nb * (fmt == TJ2_NVFP4 ? 64 : 128));
  *s16 = fmt == TJ2_FP8 ? 0 : (size_t)(rows * nb * 8);
  *s128 = (size_t)(rows * nb * 4);
  return *c + *s16 + *s128;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// 128-element chunks of a product's reduction over one or two segments.
int64_t gemm_chunks(int64_t K, int64_t K2) { return (K + 127) / 128 + (K2 + 127) / 128; }

// Carve a tj2_qtensor out of a workspace cursor.
tj2_qtensor carve(uint8_t*& cur, int fmt, int64_t rows, int64_t len) {
  size_t c, s16, s128;
  qbytes(fmt, rows, len, &c, &s16, &s128);
  tj2_qtensor q;
  q.codes = cur;
  cur += align256(c);
  q.scale16 = s16 ? cur : nullptr;
  cur += align256(s16);
  q.scale128 = reinterpret_cast<float*>(cur);
  cur += align256(s128);
  q.rows = rows;
  q.len = len;
  q.fmt = fmt;
  q.reserved = 0;
  return q;
}

size_t carve_size(int fmt, int64_t rows, int64_t len) {
  size_t c, s16, s128;
  qbytes(fmt, rows, len, &c, &s16, &s128);
  return align256(c) + align256(s16) + align256(s128);
}

QuantParams quant_params(const void* x, int x_dtype, const tj2_qtensor* x_q, int64_t rows, int64_t cols,
                         const int32_t* idx, int64_t n_idx, int grouping, int rounding, int rht, uint32_t mask,
                         uint64_t seed, uint64_t offset, const tj2_qtensor* out) {
  QuantParams p;
  memset(&p, 0, sizeof(p));
  p.in_dtype = x_dtype;
  p.x = x;
  p.ld_x = cols;
  if (x_q) p.xq = make_view(*x_q);
  p.rows = rows;
  p.cols = cols;
  p.idx = idx;
  p.n_idx = n_idx;
  p.grouping = grouping;
  p.rounding = rounding;
  p.rht = rht;
  p.rht_mask = mask & 0xFFFFu;
  p.seed = seed;
  p.offset = offset;
  p.out = make_view(*out);
  return p;
}

tj2_status run_quant(const void* x, int x_dtype, const tj2_qtensor* x_q, int64_t rows, int64_t cols,
                     const int32_t* idx, int64_t n_idx, int grouping, int rounding, int rht, uint32_t mask,
                     uint64_t seed, uint64_t offset, const tj2_qtensor* out, hipStream_t s) {
  const QuantParams p =
      quant_params(x, x_dtype, x_q, rows, cols, idx, n_idx, grouping, rounding, rht, mask, seed, offset, out);
  return hip_check(launch_quant(p, s), "quantize launch");
}

// One read of X (or W) into its NVFP4 rest columns and FP8 outlier columns.
// Rows wider than 32 KB go through the two gathering row quantizations.
// With img (the forward product's B image, rows = its output columns), the
// split quantization also writes the rows' decoded f16 values into it: NVFP4
// chunks first, then the FP8 chunks (the caller checks that the split kernel
// runs: rows within 32 KB).
SplitParams split_params(const void* x, int x_dtype, int64_t rows, int64_t K, const tj2_outlier_plan* plan,
                         const tj2_qtensor* q4, const tj2_qtensor* q8, uint8_t* img) {
  const int64_t no = plan->n_outliers, K1 = K - no;
  SplitParams p;
  memset(&p, 0, sizeof(p));
  p.in_dtype = x_dtype;
  p.x = x;
  p.rows = rows;
  p.cols = K;
  p.rest = plan->rest;
  p.outl = plan->outliers;
  p.q4 = make_view(*q4);
  p.q8 = make_view(*q8);
  if (img) {
    const int64_t tiles = (rows + 127) / 128, n0c = (K1 + 127) / 128, nch = n0c + (no + 127) / 128;
    p.img = img;
    p.img_nch = (int)nch;
    p.img_g8 = (int)n0c;
    p.img_ld = tiles * 128;
    p.img_sc = reinterpret_cast<float*>(img + (size_t)tiles * (size_t)nch * kImgChunkBytes);
  }
  return p;
}

tj2_status run_split(const void* x, int x_dtype, int64_t rows, int64_t K, const tj2_outlier_plan* plan,
                     const tj2_qtensor* q4, const tj2_qtensor* q8, hipStream_t s, uint8_t* img = nullptr) {
  const int64_t no = plan->n_outliers, K1 = K - no;
  if (K * (x_dtype == TJ2_BF16 ? 2 : 4) > 32768) {
    if (img) return fail(TJ2_ERR_ARG, "the B image needs rows within 32 KB");
    TJ2_TRY(run_quant(x, x_dtype, nullptr, rows, K, plan->rest, K1, TJ2_GROUP_ROW, TJ2_RTN, 0, 0, 0, 0, q4, s));
    return run_quant(x, x_dtype, nullptr, rows, K, plan->outliers, no, TJ2_GROUP_ROW, TJ2_RTN, 0, 0, 0, 0, q8, s);
  }
  return hip_check(launch_quant_split(split_params(x, x_dtype, rows, K, plan, q4, q8, img), s),
                   "split quantize launch");
}

// B image of a product (scratch for its f16 decode; ready = already written by
// B's producer).
struct GemmImage {
  void* ptr = nullptr;
  size_t bytes = 0;
  int ready = 0;
};

// Image bytes of a product of I x J over K (+ K2 for a second segment; 0 when
// it would not pay).
size_t image_bytes(int64_t I, int64_t J, int64_t K, int64_t K2 = 0) {
  return gemm_image_pays(I) ? align256(gemm_image_bytes(J, gemm_chunks(K, K2))) : 0;
}

// Whether the forward's product runs from a B image that the weights' split
// quantization writes beside Wq and W8: an outlier plan, the masters given and
// staged whole by that quantization (K * 4 bytes within 32 KB), an NVFP4
// segment of more than one chunk, one K split and enough row tiles.
bool fwd_image(int64_t M, int64_t N, int64_t K, int64_t no, bool w_master) {
  const int64_t K1 = K - no;
  return no > 0 && w_master && K * 4 <= 32768 && K1 > 128 && gemm_image_pays(M) &&
         gemm_split(M, N, gemm_chunks(K1, no)) == 1;
}

// Image room of a product called on its own (nvfp4_gemm): one segment, or
// two (the forward's NVFP4 and FP8 segments) when the product runs unsplit
// (the two-segment image kernel has no K split).
size_t gemm_image_room(int64_t I, int64_t J, int64_t K, int64_t K2) {
  if (K2 > 0 && (K <= 128 || gemm_split(I, J, gemm_chunks(K, K2)) != 1)) return 0;
  return image_bytes(I, J, K, K2);
}

// The image part of a product's workspace: after its split-K partials (need
// bytes, 256-aligned) when the workspace holds img_bytes more (else none).
GemmImage workspace_image(void* workspace, size_t ws_bytes, size_t need, size_t img_bytes) {
  GemmImage g;
  const uintptr_t base = reinterpret_cast<uintptr_t>(workspace);
  const size_t at = ((base + need + 255) & ~(uintptr_t)255) - base;
  if (img_bytes && ws_bytes >= at + img_bytes) {
    g.ptr = reinterpret_cast<uint8_t*>(workspace) + at;
    g.bytes = img_bytes;
  }
  return g;
}

// Point the column quantization q at the B image `img` of a product over K
// with J output columns: q's output row i is image row rows[i] (NULL: i).
void set_image(QuantParams& q, uint8_t* img, int64_t J, int64_t K, const int32_t* rows) {
  const int64_t tiles = (J + 127) / 128, nch = (K + 127) / 128;
  q.img = img;
  q.img_rows = rows;
  q.img_nch = nch;
  q.img_ld = tiles * 128;
  q.img_sc = reinterpret_cast<float*>(img + (size_t)tiles * (size_t)nch * kImgChunkBytes);
}

tj2_status run_gemm(const tj2_qtensor* A, const tj2_qtensor* B, const tj2_qtensor* A2, const tj2_qtensor* B2,
                    void* C, int c_dtype, int64_t ldc, const int32_t* col_map, int accumulate, void* ws,
                    size_t ws_bytes, hipStream_t s, const GemmImage& img = GemmImage{}) {
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.seg[0].a = make_view(*A);
  p.seg[0].b = make_view(*B);
  p.seg[0].K = A->len;
  p.nseg = 1;
  if (A2 && B2) {
    p.seg[1].a = make_view(*A2);
    p.seg[1].b = make_view(*B2);
    p.seg[1].K = A2->len;
    p.nseg = 2;
  }
  p.I = A->rows;
  p.J = B->rows;
  p.C = C;
  p.c_dtype = c_dtype;
  p.ldc = ldc;
  p.col_map = col_map;
  p.accumulate = accumulate;
  p.partial = reinterpret_cast<float*>(ws);
  p.partial_bytes = ws ? ws_bytes : 0;
  p.bimg = img.ptr;
  p.bimg_bytes = img.bytes;
  p.bimg_ready = img.ready;
  return hip_check(launch_gemm(p, s), "gemm launch");
}

// C[:, rest[j]] = A . B[j]^T and C[:, outliers[i]] = A . B8[i]^T in one product.
tj2_status run_gemm_outl(const tj2_qtensor* A, const tj2_qtensor* B, const tj2_qtensor* B8,
                         const tj2_outlier_plan* plan, void* C, int c_dtype, int64_t ldc, int accumulate, void* ws,
                         size_t ws_bytes, hipStream_t s, const GemmImage& img = GemmImage{}) {
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.seg[0].a = make_view(*A);
  p.seg[0].b = make_view(*B);
  p.seg[0].K = A->len;
  p.nseg = 1;
  p.b8 = make_view(*B8);
  p.outl = plan->outliers;
  p.rest = plan->rest;
  p.n_outl = plan->n_outliers;
  p.I = A->rows;
  p.J = B->rows + B8->rows;
  p.C = C;
  p.c_dtype = c_dtype;
  p.ldc = ldc;
  p.accumulate = accumulate;
  p.partial = reinterpret_cast<float*>(ws);
  p.partial_bytes = ws ? ws_bytes : 0;
  p.bimg = img.ptr;
  p.bimg_bytes = img.bytes;
  p.bimg_ready = img.ready;
  return hip_check(launch_gemm(p, s), "gemm launch");
}

uint32_t philox_word0(uint64_t seed, uint64_t offset) {
  uint32_t c0 = 0xFFFFFFFFu, c1 = 0xFFFFFFFFu, c2 = (uint32_t)offset, c3 = (uint32_t)(offset >> 32);
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
    uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

// Split-K workspace shared (sequentially) by the products of one backward call.
size_t bwd_gemm_ws(int64_t M, int64_t N, int64_t K1, int64_t no) {
  // with a plan, dX and dW are each one outlier-column product over all K1 + no columns
  const int64_t cn = (N + 127) / 128, cm = (M + 127) / 128;
  size_t w = gemm_workspace_bytes(M, K1 + no, cn);
  w = std::max(w, gemm_workspace_bytes(N, K1 + no, cm));
  return align256(w);
}

// Workspace of the backward with the two dY operands in format gfmt.
size_t bwd_workspace_size(int gfmt, int64_t M, int64_t N, int64_t K, int32_t n_outliers) {
  if (M <= 0 || N <= 0 || K <= 0 || n_outliers < 0 || n_outliers >= K) return 0;
  const int64_t K1 = K - n_outliers;
  size_t t = carve_size(gfmt, M, N) + carve_size(gfmt, N, M) + carve_size(TJ2_NVFP4, K1, N) +
             carve_size(TJ2_NVFP4, K1, M);
  if (n_outliers) t += carve_size(TJ2_FP8, n_outliers, N) + carve_size(TJ2_FP8, n_outliers, M);
  // the B images of dX (over N) and dW (over M), where they pay
  return t + 256 + bwd_gemm_ws(M, N, K1, n_outliers) + image_bytes(M, K, N) + image_bytes(N, K, M);
}

tj2_status check_plan(const tj2_outlier_plan* plan, int64_t K) {
  if (!plan) return TJ2_OK;
  if (!plan->outliers || !plan->rest) return fail(TJ2_ERR_ARG, "plan arrays are NULL");
  if (!aligned16(plan->outliers) || !aligned16(plan->rest)) return fail(TJ2_ERR_ALIGN, "plan arrays must be 16-byte aligned");
  if (plan->n_outliers <= 0 || plan->n_outliers % 16 || plan->n_outliers >= K)
    return fail(TJ2_ERR_SHAPE, "plan n_outliers = %d must be a positive multiple of 16 below K", plan->n_outliers);
  return TJ2_OK;
}

// Argument rules of nvfp4_gemm (and its no-allocation form).
tj2_status check_gemm(const tj2_qtensor* A, const tj2_qtensor* B, const tj2_qtensor* A2, const tj2_qtensor* B2,
                      const void* C, int32_t c_dtype, int64_t ldc, const int32_t* col_map, int32_t accumulate) {
  if (!A || !B) return fail(TJ2_ERR_ARG, "A and B are required");
  if ((A2 == nullptr) != (B2 == nullptr)) return fail(TJ2_ERR_ARG, "A2 and B2 must be given together");
  TJ2_TRY(check_qtensor(A, "A", A->fmt, A->rows, A->len));
  TJ2_TRY(check_qtensor(B, "B", B->fmt, B->rows, A->len));
  if (A2) {
    TJ2_TRY(check_qtensor(A2, "A2", A2->fmt, A->rows, A2->len));
    TJ2_TRY(check_qtensor(B2, "B2", B2->fmt, B->rows, A2->len));
  }
  if (!C) return fail(TJ2_ERR_ARG, "C is NULL");
  if (c_dtype != TJ2_F32 && c_dtype != TJ2_BF16) return fail(TJ2_ERR_ARG, "c_dtype must be TJ2_F32 or TJ2_BF16");
  if (accumulate && c_dtype != TJ2_F32) return fail(TJ2_ERR_UNSUPPORTED, "accumulate needs an fp32 output");
  if (!col_map && ldc < B->rows) return fail(TJ2_ERR_SHAPE, "ldc < J");
  if (ldc <= 0) return fail(TJ2_ERR_SHAPE, "ldc must be positive");
  if (A->rows > ((int64_t)1 << 24) * 128 || B->rows > ((int64_t)1 << 24) * 128) return fail(TJ2_ERR_SHAPE, "too many rows");
  return TJ2_OK;
}

// Scratch of nvfp4_gemm_noalloc: the split-K partial sums of one product, in a
// file-scope device array (each GPU the library runs on holds its own copy
// until the process ends).  Host code never passes the array's name to a
// kernel: it stands for a host-side shadow, not a device address.  The device
// address is looked up once per device, with that device current, and kept.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

tj2_status scratch_address(void** out) {
  int dev = -1;
  TJ2_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(TJ2_ERR_UNSUPPORTED, "device %d is beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    TJ2_TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p) return fail(TJ2_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TJ2_OK;
}

}  // namespace

extern "C" {

const char* tj2_last_error(void) { return g_err.c_str(); }

const char* tj2_version(void) { return "tj2 0.1.0 gfx950"; }

tj2_status tj2_qtensor_bytes(int32_t fmt, int64_t rows, int64_t len, size_t* codes_bytes, size_t* scale16_bytes,
                             size_t* scale128_bytes) {
  if (fmt != TJ2_NVFP4 && fmt != TJ2_FP8 && fmt != TJ2_NVFP6)
    return fail(TJ2_ERR_ARG, "format must be TJ2_NVFP4, TJ2_FP8 or TJ2_NVFP6");
  if (rows <= 0 || len <= 0 || len % 16) return fail(TJ2_ERR_SHAPE, "rows > 0 and len a positive multiple of 16 required");
  size_t c, s16, s128;
  qbytes(fmt, rows, len, &c, &s16, &s128);
  if (codes_bytes) *codes_bytes = c;
  if (scale16_bytes) *scale16_bytes = s16;
  if (scale128_bytes) *scale128_bytes = s128;
  return ok();
}

uint16_t tj2_rht_signs(uint64_t seed, uint64_t offset) { return (uint16_t)(philox_word0(seed, offset) & 0xFFFFu); }

tj2_status run_quant_dual(const void* x, int64_t rows, int64_t cols, int rht, uint64_t seed, uint64_t row_offset,
                          uint64_t col_offset, const tj2_qtensor* row_out, const tj2_qtensor* col_out, hipStream_t s) {
  DualParams d;
  d.x = reinterpret_cast<const uint16_t*>(x);
  d.rows = rows;
  d.cols = cols;
  d.row_out = make_view(*row_out);
  d.col_out = make_view(*col_out);
  d.row_mask = rht ? tj2_rht_signs(seed, row_offset) & 0xFFFFu : 0u;
  d.col_mask = rht ? tj2_rht_signs(seed, col_offset) & 0xFFFFu : 0u;
  d.seed = seed;
  d.row_offset = row_offset;
  d.col_offset = col_offset;
  d.rht = rht ? 1 : 0;
  return hip_check(launch_quant_dual(d, s), "dual quantize launch");
}

tj2_status nvfp4_quantize_dual(const void* x, int64_t rows, int64_t cols, int32_t rht, uint64_t seed,
                               uint64_t row_offset, uint64_t col_offset, tj2_qtensor* row_out, tj2_qtensor* col_out,
                               void* stream) {
  if (!x || !row_out || !col_out) return fail(TJ2_ERR_ARG, "x, row_out and col_out are required");
  if (!aligned16(x)) return fail(TJ2_ERR_ALIGN, "x must be 16-byte aligned");
  if (rows <= 0 || cols <= 0) return fail(TJ2_ERR_SHAPE, "rows and cols must be positive");
  if (rows > (int64_t)1 << 30 || cols > (int64_t)1 << 30) return fail(TJ2_ERR_SHAPE, "dimension too large");
  if (rows % 16 || cols % 16) return fail(TJ2_ERR_SHAPE, "rows and cols must be multiples of 16");
  if (row_out->fmt != TJ2_NVFP4 && row_out->fmt != TJ2_NVFP6)
    return fail(TJ2_ERR_ARG, "outputs must be NVFP4 or NVFP6");
  if (col_out->fmt != row_out->fmt) return fail(TJ2_ERR_ARG, "row_out and col_out must have the same format");
  TJ2_TRY(check_qtensor(row_out, "row_out", row_out->fmt, rows, cols));
  TJ2_TRY(check_qtensor(col_out, "col_out", col_out->fmt, cols, rows));
  if (((rows + 127) / 128) * ((cols + 127) / 128) >= ((int64_t)1 << 31)) return fail(TJ2_ERR_SHAPE, "tensor too large for one launch");
  return run_quant_dual(x, rows, cols, rht, seed, row_offset, col_offset, row_out, col_out, (hipStream_t)stream) == TJ2_OK
             ? ok() : TJ2_ERR_HIP;
}

tj2_status nvfp4_quantize(const void* x, int32_t x_dtype, const tj2_qtensor* x_q, int64_t rows, int64_t cols,
                          const int32_t* col_idx, int64_t n_idx, int32_t grouping, int32_t rounding, int32_t rht,
                          uint32_t rht_signs, uint64_t seed, uint64_t offset, tj2_qtensor* out, void* stream) {
  if (grouping != TJ2_GROUP_ROW && grouping != TJ2_GROUP_COL) return fail(TJ2_ERR_ARG, "bad grouping %d", grouping);
  if (rounding != TJ2_RTN && rounding != TJ2_SR) return fail(TJ2_ERR_ARG, "bad rounding %d", rounding);
  if (!out) return fail(TJ2_ERR_ARG, "out is NULL");
  if (out->fmt != TJ2_NVFP4 && out->fmt != TJ2_FP8 && out->fmt != TJ2_NVFP6)
    return fail(TJ2_ERR_ARG, "out format must be NVFP4, FP8 or NVFP6");
  if (rows <= 0 || cols <= 0) return fail(TJ2_ERR_SHAPE, "rows and cols must be positive");
  if (rows > (int64_t)1 << 30 || cols > (int64_t)1 << 30) return fail(TJ2_ERR_SHAPE, "dimension too large");
  const bool dense = x_dtype == TJ2_BF16 || x_dtype == TJ2_F32;
  if (dense) {
    if (!x) return fail(TJ2_ERR_ARG, "x is NULL");
    if (!aligned16(x)) return fail(TJ2_ERR_ALIGN, "x must be 16-byte aligned");
  } else if (x_dtype == TJ2_NVFP4 || x_dtype == TJ2_FP8) {
    TJ2_TRY(check_qtensor(x_q, "x_q", x_dtype, rows, cols));
  } else {
    return fail(TJ2_ERR_ARG, "bad x_dtype %d", x_dtype);
  }
  if (out->fmt == TJ2_NVFP6 && !dense) return fail(TJ2_ERR_UNSUPPORTED, "NVFP6 output needs a dense (bf16 / fp32) input");
  if (col_idx) {
    if (out->fmt == TJ2_NVFP6) return fail(TJ2_ERR_UNSUPPORTED, "col_idx with an NVFP6 output is not implemented");
    if (grouping != TJ2_GROUP_ROW || !dense) return fail(TJ2_ERR_UNSUPPORTED, "col_idx needs row grouping and a dense input");
    if (!aligned16(col_idx)) return fail(TJ2_ERR_ALIGN, "col_idx must be 16-byte aligned");
    if (n_idx <= 0 || n_idx % 16 || n_idx > cols) return fail(TJ2_ERR_SHAPE, "n_idx must be a positive multiple of 16 <= cols");
  }
  if (grouping == TJ2_GROUP_ROW) {
    if (!dense) return fail(TJ2_ERR_UNSUPPORTED, "row grouping of a quantized input is not implemented");
    const int64_t n = col_idx ? n_idx : cols;
    if (n % 16) return fail(TJ2_ERR_SHAPE, "grouped length %lld is not a multiple of 16", (long long)n);
    if (cols % 8) return fail(TJ2_ERR_SHAPE, "cols must be a multiple of 8");
    TJ2_TRY(check_qtensor(out, "out", out->fmt, rows, n));
    const int64_t nb = (n + 127) / 128;
    if (rows * nb * 8 >= ((int64_t)1 << 31)) return fail(TJ2_ERR_SHAPE, "tensor too large for one launch");
  } else {
    if (rows % 16 || cols % 16) return fail(TJ2_ERR_SHAPE, "column grouping needs rows and cols multiples of 16");
    TJ2_TRY(check_qtensor(out, "out", out->fmt, cols, rows));
  }
  return run_quant(x, x_dtype, x_q, rows, cols, col_idx, n_idx, grouping, rounding, rht ? 1 : 0, rht_signs, seed,
                   offset, out, (hipStream_t)stream) == TJ2_OK ? ok() : TJ2_ERR_HIP;
}

size_t nvfp4_gemm_workspace_size(int64_t I, int64_t J, int64_t K, int64_t K2) {
  if (I <= 0 || J <= 0 || K <= 0 || K2 < 0) return 0;
  const size_t part = gemm_workspace_bytes(I, J, gemm_chunks(K, K2));
  const size_t img = gemm_image_room(I, J, K, K2);
  return img ? align256(part) + img : part;
}

tj2_status nvfp4_gemm(const tj2_qtensor* A, const tj2_qtensor* B, const tj2_qtensor* A2, const tj2_qtensor* B2,
                      void* C, int32_t c_dtype, int64_t ldc, const int32_t* col_map, int32_t accumulate,
                      void* workspace, size_t ws_bytes, void* stream) {
  TJ2_TRY(check_gemm(A, B, A2, B2, C, c_dtype, ldc, col_map, accumulate));
  GemmImage img;
  if (workspace) {
    if (!aligned16(workspace)) return fail(TJ2_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t need = gemm_workspace_bytes(A->rows, B->rows, gemm_chunks(A->len, A2 ? A2->len : 0));
    if (ws_bytes < need) return fail(TJ2_ERR_ARG, "workspace of %zu bytes required (got %zu)", need, ws_bytes);
    img = workspace_image(workspace, ws_bytes, need, gemm_image_room(A->rows, B->rows, A->len, A2 ? A2->len : 0));
  }
  return run_gemm(A, B, A2, B2, C, c_dtype, ldc, col_map, accumulate, workspace, workspace ? ws_bytes : 0,
                  (hipStream_t)stream, img) == TJ2_OK ? ok() : TJ2_ERR_HIP;
}

tj2_status nvfp4_gemm_noalloc(const tj2_qtensor* A, const tj2_qtensor* B, const tj2_qtensor* A2,
                              const tj2_qtensor* B2, void* C, int32_t c_dtype, int64_t ldc, const int32_t* col_map,
                              int32_t accumulate, void* stream) {
  TJ2_TRY(check_gemm(A, B, A2, B2, C, c_dtype, ldc, col_map, accumulate));
  const size_t need = gemm_workspace_bytes(A->rows, B->rows, gemm_chunks(A->len, A2 ? A2->len : 0));
  if (need > kScratchBytes)
    return fail(TJ2_ERR_SHAPE, "the K split of this product needs %zu bytes of scratch; nvfp4_gemm_noalloc holds %zu",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need) TJ2_TRY(scratch_address(&ws));
  return run_gemm(A, B, A2, B2, C, c_dtype, ldc, col_map, accumulate, ws, ws ? kScratchBytes : 0,
                  (hipStream_t)stream) == TJ2_OK ? ok() : TJ2_ERR_HIP;
}

tj2_status nvfp4_gemm_outlier_cols(const tj2_qtensor* A, const tj2_qtensor* B, const tj2_qtensor* B8,
                                   const tj2_outlier_plan* plan, void* C, int32_t c_dtype, int64_t ldc,
                                   int32_t accumulate, void* workspace, size_t ws_bytes, void* stream) {
  if (!A || !B || !B8 || !plan) return fail(TJ2_ERR_ARG, "A, B, B8 and plan are required");
  if (workspace && !aligned16(workspace)) return fail(TJ2_ERR_ALIGN, "workspace must be 16-byte aligned");
  if ((A->fmt != TJ2_NVFP4 && A->fmt != TJ2_NVFP6) || B->fmt != TJ2_NVFP4 || B8->fmt != TJ2_FP8)
    return fail(TJ2_ERR_UNSUPPORTED, "A must be NVFP4 or NVFP6, B NVFP4, B8 FP8");
  const int64_t J = B->rows + B8->rows;
  TJ2_TRY(check_plan(plan, J));
  if (plan->n_outliers != B8->rows) return fail(TJ2_ERR_SHAPE, "B8 rows (%lld) != n_outliers (%d)", (long long)B8->rows, plan->n_outliers);
  TJ2_TRY(check_qtensor(A, "A", A->fmt, A->rows, A->len));
  TJ2_TRY(check_qtensor(B, "B", TJ2_NVFP4, B->rows, A->len));
  TJ2_TRY(check_qtensor(B8, "B8", TJ2_FP8, B8->rows, A->len));
  if (!C) return fail(TJ2_ERR_ARG, "C is NULL");
  if (c_dtype != TJ2_F32 && c_dtype != TJ2_BF16) return fail(TJ2_ERR_ARG, "c_dtype must be TJ2_F32 or TJ2_BF16");
  if (accumulate && c_dtype != TJ2_F32) return fail(TJ2_ERR_UNSUPPORTED, "accumulate needs an fp32 output");
  if (ldc < J) return fail(TJ2_ERR_SHAPE, "ldc < J");
  if (A->rows > ((int64_t)1 << 24) * 128 || J > ((int64_t)1 << 24) * 128) return fail(TJ2_ERR_SHAPE, "too many rows");
  GemmImage img;
  if (workspace) {
    const size_t need = gemm_workspace_bytes(A->rows, J, gemm_chunks(A->len, 0));
    if (ws_bytes < need) return fail(TJ2_ERR_ARG, "workspace of %zu bytes required (got %zu)", need, ws_bytes);
    img = workspace_image(workspace, ws_bytes, need, image_bytes(A->rows, J, A->len));
  }
  return run_gemm_outl(A, B, B8, plan, C, c_dtype, ldc, accumulate, workspace, workspace ? ws_bytes : 0,
                       (hipStream_t)stream, img) == TJ2_OK ? ok() : TJ2_ERR_HIP;
}

size_t nvfp4_linear_fwd_workspace_size(int64_t M, int64_t N, int64_t K, int32_t n_outliers) {
  if (M <= 0 || N <= 0 || K <= 0 || n_outliers < 0 || n_outliers >= K) return 0;
  const size_t part = gemm_workspace_bytes(M, N, gemm_chunks(K - n_outliers, n_outliers));
  const size_t img = fwd_image(M, N, K, n_outliers, true) ? image_bytes(M, N, K - n_outliers, n_outliers) : 0;
  return img ? align256(part) + img : part;
}

tj2_status nvfp4_linear_fwd(const void* X, int64_t M, int64_t K, int64_t N, const float* W_master, tj2_qtensor* Wq,
                            tj2_qtensor* W8, const tj2_outlier_plan* plan, tj2_qtensor* Xq, tj2_qtensor* X8, void* Y,
                            int32_t y_dtype, void* workspace, size_t ws_bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  TJ2_TRY(check_dims(M, "M"));
  TJ2_TRY(check_dims(K, "K"));
  TJ2_TRY(check_dims(N, "N"));
  if (!X || !Y) return fail(TJ2_ERR_ARG, "X and Y are required");
  if (!aligned16(X) || !aligned16(Y) || (W_master && !aligned16(W_master))) return fail(TJ2_ERR_ALIGN, "X, Y, W_master must be 16-byte aligned");
  if (y_dtype != TJ2_BF16 && y_dtype != TJ2_F32) return fail(TJ2_ERR_ARG, "y_dtype must be TJ2_BF16 or TJ2_F32");
  TJ2_TRY(check_plan(plan, K));
  const int64_t no = plan ? plan->n_outliers : 0;
  const int64_t K1 = K - no;
  TJ2_TRY(check_qtensor(Xq, "Xq", TJ2_NVFP4, M, K1));
  TJ2_TRY(check_qtensor(Wq, "Wq", TJ2_NVFP4, N, K1));
  if (plan) {
    TJ2_TRY(check_qtensor(X8, "X8", TJ2_FP8, M, no));
    TJ2_TRY(check_qtensor(W8, "W8", TJ2_FP8, N, no));
  }
  GemmImage img;
  if (workspace) {
    if (!aligned16(workspace)) return fail(TJ2_ERR_ALIGN, "workspace must be 16-byte aligned");
    // the K-split partials are required; the B image is used when there is room for it
    const size_t need = gemm_workspace_bytes(M, N, gemm_chunks(K1, no));
    if (ws_bytes < need) return fail(TJ2_ERR_ARG, "workspace of %zu bytes required (got %zu)", need, ws_bytes);
    if (fwd_image(M, N, K, no, W_master != nullptr))
      img = workspace_image(workspace, ws_bytes, need, image_bytes(M, N, K1, no));
  }
  if (plan) {
    uint8_t* wimg = static_cast<uint8_t*>(img.ptr);
    if (W_master && K * 4 <= 32768) {
      // X and the masters split in one launch (the masters also write the product's image)
      TJ2_TRY(hip_check(launch_quant_split2(split_params(X, TJ2_BF16, M, K, plan, Xq, X8, nullptr),
                                            split_params(W_master, TJ2_F32, N, K, plan, Wq, W8, wimg), s),
                        "split quantize launch"));
    } else {
      TJ2_TRY(run_split(X, TJ2_BF16, M, K, plan, Xq, X8, s));
      if (W_master) TJ2_TRY(run_split(W_master, TJ2_F32, N, K, plan, Wq, W8, s, wimg));
    }
    img.ready = img.ptr ? 1 : 0;  // written by the split quantization above
  } else {
    TJ2_TRY(run_quant(X, TJ2_BF16, nullptr, M, K, nullptr, K1, TJ2_GROUP_ROW, TJ2_RTN, 0, 0, 0, 0, Xq, s));
    if (W_master) TJ2_TRY(run_quant(W_master, TJ2_F32, nullptr, N, K, nullptr, K1, TJ2_GROUP_ROW, TJ2_RTN, 0, 0, 0, 0, Wq, s));
  }
  TJ2_TRY(run_gemm(Xq, Wq, plan ? X8 : nullptr, plan ? W8 : nullptr, Y, y_dtype, N, nullptr, 0, workspace,
                   workspace ? ws_bytes : 0, s, img));
  return ok();
}

size_t nvfp4_linear_bwd_workspace_size(int64_t M, int64_t N, int64_t K, int32_t n_outliers) {
  return bwd_workspace_size(TJ2_NVFP4, M, N, K, n_outliers);
}

}  // extern "C"

namespace {

// The backward of nvfp4_linear_bwd with the two dY operands in format gfmt
// (TJ2_NVFP4, or TJ2_NVFP6 for the FP6 x FP4 variant).
tj2_status linear_bwd_impl(int gfmt, const void* dY, int64_t M, int64_t N, int64_t K, const tj2_qtensor* Xq,
                           const tj2_qtensor* X8, const tj2_qtensor* Wq, const tj2_qtensor* W8,
                           const tj2_outlier_plan* plan, int32_t rht, uint64_t seed, uint64_t offset, void* dX,
                           int32_t dx_dtype, float* dW, tj2_bwd_operands* ops, void* workspace, size_t ws_bytes,
                           void* stream) {
  hipStream_t s = (hipStream_t)stream;
  TJ2_TRY(check_dims(M, "M"));
  TJ2_TRY(check_dims(K, "K"));
  TJ2_TRY(check_dims(N, "N"));
  if (!dY || !dX || !dW) return fail(TJ2_ERR_ARG, "dY, dX and dW are required");
  if (!aligned16(dY) || !aligned16(dX) || !aligned16(dW)) return fail(TJ2_ERR_ALIGN, "dY, dX, dW must be 16-byte aligned");
  if (dx_dtype != TJ2_BF16 && dx_dtype != TJ2_F32) return fail(TJ2_ERR_ARG, "dx_dtype must be TJ2_BF16 or TJ2_F32");
  TJ2_TRY(check_plan(plan, K));
  const int64_t no = plan ? plan->n_outliers : 0;
  const int64_t K1 = K - no;
  TJ2_TRY(check_qtensor(Xq, "Xq", TJ2_NVFP4, M, K1));
  TJ2_TRY(check_qtensor(Wq, "Wq", TJ2_NVFP4, N, K1));
  if (plan) {
    TJ2_TRY(check_qtensor(X8, "X8", TJ2_FP8, M, no));
    TJ2_TRY(check_qtensor(W8, "W8", TJ2_FP8, N, no));
  }
  tj2_bwd_operands local;
  tj2_bwd_operands* o = ops;
  const size_t gws = bwd_gemm_ws(M, N, K1, no);
  // B images of the two products (dX: Wt / W8t over N; dW: Xt / X8t over M),
  // written by the column quantization below
  const size_t idx_bytes = image_bytes(M, K, N), idw_bytes = image_bytes(N, K, M);
  void* gemm_ws = nullptr;
  GemmImage img_dx, img_dw;
  auto carve_images = [&](uint8_t*& cur) {
    if (idx_bytes) img_dx = GemmImage{cur, idx_bytes, 1};
    cur += idx_bytes;
    if (idw_bytes) img_dw = GemmImage{cur, idw_bytes, 1};
    cur += idw_bytes;
  };
  if (!o) {
    const size_t need = bwd_workspace_size(gfmt, M, N, K, (int32_t)no);
    if (!workspace || ws_bytes < need)
      return fail(TJ2_ERR_ARG, "workspace of %zu bytes required (got %zu)", need, ws_bytes);
    uint8_t* cur = reinterpret_cast<uint8_t*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~(uintptr_t)255);
    gemm_ws = gws ? cur : nullptr;
    cur += gws;
    carve_images(cur);
    memset(&local, 0, sizeof(local));
    local.dYq = carve(cur, gfmt, M, N);
    local.dYt = carve(cur, gfmt, N, M);
    local.Wt = carve(cur, TJ2_NVFP4, K1, N);
    local.Xt = carve(cur, TJ2_NVFP4, K1, M);
    if (plan) {
      local.W8t = carve(cur, TJ2_FP8, no, N);
      local.X8t = carve(cur, TJ2_FP8, no, M);
    }
    o = &local;
  } else {
    if (workspace && ws_bytes >= gws && aligned16(workspace)) gemm_ws = gws ? workspace : nullptr;
    // images too when the workspace holds them after the split-K partials
    const uintptr_t base = reinterpret_cast<uintptr_t>(workspace);
    const uintptr_t img0 = (base + gws + 255) & ~(uintptr_t)255;
    if (workspace && aligned16(workspace) && img0 + idx_bytes + idw_bytes <= base + ws_bytes) {
      uint8_t* cur = reinterpret_cast<uint8_t*>(img0);
      carve_images(cur);
    }
    TJ2_TRY(check_qtensor(&o->dYq, "ops.dYq", gfmt, M, N));
    TJ2_TRY(check_qtensor(&o->dYt, "ops.dYt", gfmt, N, M));
    TJ2_TRY(check_qtensor(&o->Wt, "ops.Wt", TJ2_NVFP4, K1, N));
    TJ2_TRY(check_qtensor(&o->Xt, "ops.Xt", TJ2_NVFP4, K1, M));
    if (plan) {
      TJ2_TRY(check_qtensor(&o->W8t, "ops.W8t", TJ2_FP8, no, N));
      TJ2_TRY(check_qtensor(&o->X8t, "ops.X8t", TJ2_FP8, no, M));
    }
  }
  const int r = rht ? 1 : 0;
  const uint32_t mdx = r ? tj2_rht_signs(seed, offset + 0) : 0u;
  const uint32_t mdw = r ? tj2_rht_signs(seed, offset + 2) : 0u;
  // dY once into both groupings: dYq along N (dX signs, draws at offset + 0) and
  // dY^T q along M (dW signs, offset + 2)
  TJ2_TRY(run_quant_dual(dY, M, N, r, seed, offset + 0, offset + 2, &o->dYq, &o->dYt, s));
  // the other column (re-grouped, transposed) operands of both products in one
  // launch, the small FP8 slices first so their latency hides behind the large ones
  QuantParams cols[kColMultiMax];
  int nc = 0;
  const bool w_given = ops && ops->w_given;  // the re-grouped weights come from the master pass
  // the images: output row i of Wt / Xt is column rest[i] of the products'
  // outputs, row i of W8t / X8t column outliers[i]
  const int32_t* rest_rows = plan ? plan->rest : nullptr;
  const int32_t* outl_rows = plan ? plan->outliers : nullptr;
  if (plan) {
    cols[nc] = quant_params(nullptr, TJ2_FP8, X8, M, no, nullptr, 0, TJ2_GROUP_COL, TJ2_SR, r, mdw, seed, offset + 5, &o->X8t);
    if (img_dw.ptr) set_image(cols[nc], (uint8_t*)img_dw.ptr, K, M, outl_rows);
    ++nc;
    if (!w_given) {
      cols[nc] = quant_params(nullptr, TJ2_FP8, W8, N, no, nullptr, 0, TJ2_GROUP_COL, TJ2_SR, r, mdx, seed, offset + 4, &o->W8t);
      if (img_dx.ptr) set_image(cols[nc], (uint8_t*)img_dx.ptr, K, N, outl_rows);
      ++nc;
    }
  }
  if (!w_given) {
    cols[nc] = quant_params(nullptr, TJ2_NVFP4, Wq, N, K1, nullptr, 0, TJ2_GROUP_COL, TJ2_SR, r, mdx, seed, offset + 1, &o->Wt);
    if (img_dx.ptr) set_image(cols[nc], (uint8_t*)img_dx.ptr, K, N, rest_rows);
    ++nc;
  } else {
    img_dx.ready = 0;  // the re-grouped weights were given: the product decodes its image
  }
  cols[nc] = quant_params(nullptr, TJ2_NVFP4, Xq, M, K1, nullptr, 0, TJ2_GROUP_COL, TJ2_SR, r, mdw, seed, offset + 3, &o->Xt);
  if (img_dw.ptr) set_image(cols[nc], (uint8_t*)img_dw.ptr, K, M, rest_rows);
  ++nc;
  TJ2_TRY(hip_check(launch_quant_col_multi(cols, nc, s), "column quantize launch"));
  if (!plan) {
    TJ2_TRY(run_gemm(&o->dYq, &o->Wt, nullptr, nullptr, dX, dx_dtype, K, nullptr, 0, gemm_ws, gws, s, img_dx));
    TJ2_TRY(run_gemm(&o->dYt, &o->Xt, nullptr, nullptr, dW, TJ2_F32, K, nullptr, 0, gemm_ws, gws, s, img_dw));
    return ok();
  }
  TJ2_TRY(run_gemm_outl(&o->dYq, &o->Wt, &o->W8t, plan, dX, dx_dtype, K, 0, gemm_ws, gws, s, img_dx));
  TJ2_TRY(run_gemm_outl(&o->dYt, &o->Xt, &o->X8t, plan, dW, TJ2_F32, K, 0, gemm_ws, gws, s, img_dw));
  return ok();
}

}  // namespace

extern "C" {

tj2_status nvfp4_linear_bwd(const void* dY, int64_t M, int64_t N, int64_t K, const tj2_qtensor* Xq,
                            const tj2_qtensor* X8, const tj2_qtensor* Wq, const tj2_qtensor* W8,
                            const tj2_outlier_plan* plan, int32_t rht, uint64_t seed, uint64_t offset, void* dX,
                            int32_t dx_dtype, float* dW, tj2_bwd_operands* ops, void* workspace, size_t ws_bytes,
                            void* stream) {
  return linear_bwd_impl(TJ2_NVFP4, dY, M, N, K, Xq, X8, Wq, W8, plan, rht, seed, offset, dX, dx_dtype, dW, ops,
                         workspace, ws_bytes, stream);
}

size_t nvfp6x4_linear_bwd_workspace_size(int64_t M, int64_t N, int64_t K, int32_t n_outliers) {
  return bwd_workspace_size(TJ2_NVFP6, M, N, K, n_outliers);
}

tj2_status nvfp6x4_linear_bwd(const void* dY, int64_t M, int64_t N, int64_t K, const tj2_qtensor* Xq,
                              const tj2_qtensor* X8, const tj2_qtensor* Wq, const tj2_qtensor* W8,
                              const tj2_outlier_plan* plan, int32_t rht, uint64_t seed, uint64_t offset, void* dX,
                              int32_t dx_dtype, float* dW, tj2_bwd_operands* ops, void* workspace, size_t ws_bytes,
                              void* stream) {
  return linear_bwd_impl(TJ2_NVFP6, dY, M, N, K, Xq, X8, Wq, W8, plan, rht, seed, offset, dX, dx_dtype, dW, ops,
                         workspace, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Checked per-matrix parameters of OsciReset / the fused master pass.
tj2_status osci_problem(float* W, float* W_prev, float* m, float* v, const float* grad, float* Q_prev, float* dQ,
                        float* dM, int64_t N, int64_t K, bool master, const tj2_outlier_plan* plan,
                        tj2_qtensor* Wq_out, tj2_qtensor* W8_out, OsciProblem* out) {
  if (!W || !Q_prev || !dQ || !dM || (master ? (!m || !v || !grad) : !W_prev))
    return fail(TJ2_ERR_ARG, master ? "W, m, v, grad and the state arrays are required"
                                    : "W and the state arrays are required");
  if (!aligned16(W) || !aligned16(Q_prev) || !aligned16(dQ) || !aligned16(dM) ||
      (master ? (!aligned16(m) || !aligned16(v) || !aligned16(grad)) : !aligned16(W_prev)))
    return fail(TJ2_ERR_ALIGN, "arrays must be 16-byte aligned");
  if (N <= 0 || N > ((int64_t)1 << 30)) return fail(TJ2_ERR_SHAPE, "N must be positive");
  TJ2_TRY(check_dims(K, "K"));
  TJ2_TRY(check_plan(plan, K));
  const int64_t no = plan ? plan->n_outliers : 0, K1 = K - no;
  const int64_t hpr1 = (K1 + 127) / 128 * 16, hpr = hpr1 + (no + 127) / 128 * 16;  // half groups per row
  if (N * hpr >= ((int64_t)1 << 31)) return fail(TJ2_ERR_SHAPE, "tensor too large for one launch");
  if (W8_out && !plan) return fail(TJ2_ERR_ARG, "W8_out needs an outlier plan");
  OsciProblem& p = *out;
  memset(&p, 0, sizeof(p));
  p.W = W; p.W_prev = W_prev; p.Q_prev = Q_prev; p.dQ = dQ; p.dM = dM;
  p.m = m; p.v = v; p.grad = grad;
  p.N = (int32_t)N; p.K = (int32_t)K;
  p.rest = plan ? plan->rest : nullptr;
  p.outl = plan ? plan->outliers : nullptr;
  p.K1 = (int32_t)K1; p.no = (int32_t)no;
  p.hpr = (int32_t)hpr; p.hpr1 = (int32_t)hpr1;
  if (Wq_out) TJ2_TRY(check_qtensor(Wq_out, "Wq_out", TJ2_NVFP4, N, K1));
  if (W8_out) TJ2_TRY(check_qtensor(W8_out, "W8_out", TJ2_FP8, N, no));
  p.wq = make_qout(Wq_out);
  p.w8 = make_qout(W8_out);
  return TJ2_OK;
}

tj2_status osci_shared(int32_t mode, float tau, int32_t reset_enabled, bool master, uint64_t* reset_count,
                       const tj2_osci_diag* diag, const tj2_adamw_params* adam, OsciShared* out) {
  if (master) {
    if (!adam) return fail(TJ2_ERR_ARG, "adam parameters are required");
    if (mode != TJ2_OSCI_ACCUM && mode != TJ2_OSCI_WINDOW_END) return fail(TJ2_ERR_ARG, "mode must be ACCUM or WINDOW_END");
  } else if (mode != TJ2_OSCI_INIT && mode != TJ2_OSCI_ACCUM && mode != TJ2_OSCI_WINDOW_END) {
    return fail(TJ2_ERR_ARG, "bad mode %d", mode);
  }
  if (!(tau >= 0.0f)) return fail(TJ2_ERR_ARG, "tau must be >= 0");
  OsciShared& c = *out;
  memset(&c, 0, sizeof(c));
  c.mode = mode;
  c.tau = tau;
  c.reset_enabled = reset_enabled ? 1 : 0;
  if (master) {
    c.lr = adam->lr; c.beta1 = adam->beta1; c.beta2 = adam->beta2; c.eps = adam->eps;
    c.weight_decay = adam->weight_decay; c.bc1 = adam->bias_correction1; c.bc2 = adam->bias_correction2;
  }
  c.reset_count = reinterpret_cast<unsigned long long*>(reset_count);
  return diag_pointers(diag, &c.flips, &c.risk_hist);
}

// The next backward's re-grouped weight operands from the codes the pass wrote:
// W-hat grouped along N (RHT with the dX mask, SR at offset + 1) and its FP8
// outlier rows (offset + 4), exactly as nvfp4_linear_bwd would form them.
tj2_status check_next(const tj2_next_bwd* nx, const OsciProblem& p, const tj2_qtensor* Wq_out,
                      const tj2_qtensor* W8_out) {
  if (!nx) return TJ2_OK;
  if (!nx->Wt) return fail(TJ2_ERR_ARG, "next->Wt is required");
  if (!Wq_out || (p.rest && !W8_out)) return fail(TJ2_ERR_ARG, "next needs Wq_out (and W8_out with a plan)");
  if (p.N % 16) return fail(TJ2_ERR_SHAPE, "next: N = %d must be a multiple of 16 for the re-grouping", p.N);
  TJ2_TRY(check_qtensor(nx->Wt, "next->Wt", TJ2_NVFP4, p.K1, p.N));
  if (p.rest) TJ2_TRY(check_qtensor(nx->W8t, "next->W8t", TJ2_FP8, p.no, p.N));
  return TJ2_OK;
}

tj2_status launch_next(const std::vector<const tj2_next_bwd*>& nexts, const std::vector<const tj2_qtensor*>& wqs,
                       const std::vector<const tj2_qtensor*>& w8s, hipStream_t s) {
  std::vector<QuantParams> qp[2];  // by Hadamard switch (one launch shares it)
  for (size_t i = 0; i < nexts.size(); ++i) {
    const tj2_next_bwd* nx = nexts[i];
    if (!nx) continue;
    const int r = nx->rht ? 1 : 0;
    const uint32_t mdx = r ? tj2_rht_signs(nx->seed, nx->offset + 0) : 0u;
    const tj2_qtensor* wq = wqs[i];
    qp[r].push_back(quant_params(nullptr, TJ2_NVFP4, wq, wq->rows, wq->len, nullptr, 0, TJ2_GROUP_COL, TJ2_SR, r, mdx,
                                 nx->seed, nx->offset + 1, nx->Wt));
    if (w8s[i])
      qp[r].push_back(quant_params(nullptr, TJ2_FP8, w8s[i], w8s[i]->rows, w8s[i]->len, nullptr, 0, TJ2_GROUP_COL,
                                   TJ2_SR, r, mdx, nx->seed, nx->offset + 4, nx->W8t));
  }
  for (int r = 0; r < 2; ++r)
    for (size_t i = 0; i < qp[r].size(); i += kColMultiMax) {
      const int cnt = (int)std::min<size_t>(kColMultiMax, qp[r].size() - i);
      TJ2_TRY(hip_check(launch_quant_col_multi(qp[r].data() + i, cnt, s), "re-grouping launch"));
    }
  return TJ2_OK;
}

tj2_status run_osci(const OsciShared& c, const std::vector<OsciProblem>& ps, bool master, hipStream_t s) {
  for (size_t i = 0; i < ps.size(); i += kOsciMultiMax) {
    const int cnt = (int)std::min<size_t>(kOsciMultiMax, ps.size() - i);
    TJ2_TRY(hip_check(launch_osci_multi(c, ps.data() + i, cnt, master, s), master ? "master update launch" : "osci launch"));
  }
  return TJ2_OK;
}

}  // namespace

extern "C" {

tj2_status master_update_step(float* W, float* m, float* v, const float* grad, float* Q_prev, float* dQ, float* dM,
                              int64_t N, int64_t K, const tj2_adamw_params* adam, int32_t mode, float tau,
                              int32_t reset_enabled, const tj2_outlier_plan* plan, tj2_qtensor* Wq_out,
                              tj2_qtensor* W8_out, const tj2_next_bwd* next, uint64_t* reset_count,
                              const tj2_osci_diag* diag, void* stream) {
  tj2_master_tensor t;
  memset(&t, 0, sizeof(t));
  t.W = W; t.m = m; t.v = v; t.grad = grad; t.Q_prev = Q_prev; t.dQ = dQ; t.dM = dM; t.N = N; t.K = K;
  t.Wq_out = Wq_out; t.plan = plan; t.W8_out = W8_out; t.next = next;
  const tj2_status st = master_update_step_multi(&t, 1, adam, mode, tau, reset_enabled, reset_count, diag, stream);
  if (st != TJ2_OK && strncmp(tj2_last_error(), "tensors[0]: ", 12) == 0) g_err = g_err.substr(12);
  return st;
}

tj2_status master_update_step_multi(const tj2_master_tensor* tensors, int32_t n, const tj2_adamw_params* adam,
                                    int32_t mode, float tau, int32_t reset_enabled, uint64_t* reset_count,
                                    const tj2_osci_diag* diag, void* stream) {
  if (!tensors || n < 1) return fail(TJ2_ERR_ARG, "tensors must list at least one matrix");
  OsciShared c;
  TJ2_TRY(osci_shared(mode, tau, reset_enabled, true, reset_count, diag, adam, &c));
  std::vector<OsciProblem> ps((size_t)n);
  std::vector<const tj2_next_bwd*> nexts((size_t)n);
  std::vector<const tj2_qtensor*> wqs((size_t)n), w8s((size_t)n);
  bool any_next = false;
  for (int32_t i = 0; i < n; ++i) {
    const tj2_master_tensor& x = tensors[i];
    tj2_status st = osci_problem(x.W, nullptr, x.m, x.v, x.grad, x.Q_prev, x.dQ, x.dM, x.N, x.K, true, x.plan,
                                 x.Wq_out, x.W8_out, &ps[(size_t)i]);
    if (st == TJ2_OK) st = check_next(x.next, ps[(size_t)i], x.Wq_out, x.W8_out);
    if (st != TJ2_OK) return fail(st, "tensors[%d]: %s", i, std::string(tj2_last_error()).c_str());
    nexts[(size_t)i] = x.next;
    wqs[(size_t)i] = x.Wq_out;
    w8s[(size_t)i] = x.plan ? x.W8_out : nullptr;
    any_next = any_next || x.next;
  }
  TJ2_TRY(run_osci(c, ps, true, (hipStream_t)stream));
  if (any_next) TJ2_TRY(launch_next(nexts, wqs, w8s, (hipStream_t)stream));
  return ok();
}

tj2_status osci_reset_step(float* W, float* W_prev, float* Q_prev, float* dQ, float* dM, int64_t N, int64_t K,
                           int32_t mode, float tau, int32_t reset_enabled, const tj2_outlier_plan* plan,
                           tj2_qtensor* Wq_out, tj2_qtensor* W8_out, uint64_t* reset_count,
                           const tj2_osci_diag* diag, void* stream) {
  tj2_osci_tensor t;
  memset(&t, 0, sizeof(t));
  t.W = W; t.W_prev = W_prev; t.Q_prev = Q_prev; t.dQ = dQ; t.dM = dM; t.N = N; t.K = K;
  t.Wq_out = Wq_out; t.plan = plan; t.W8_out = W8_out;
  const tj2_status st = osci_reset_step_multi(&t, 1, mode, tau, reset_enabled, reset_count, diag, stream);
  if (st != TJ2_OK && strncmp(tj2_last_error(), "tensors[0]: ", 12) == 0) g_err = g_err.substr(12);
  return st;
}

tj2_status osci_reset_step_multi(const tj2_osci_tensor* tensors, int32_t n, int32_t mode, float tau,
                                 int32_t reset_enabled, uint64_t* reset_count, const tj2_osci_diag* diag,
                                 void* stream) {
  if (!tensors || n < 1) return fail(TJ2_ERR_ARG, "tensors must list at least one matrix");
  OsciShared c;
  TJ2_TRY(osci_shared(mode, tau, reset_enabled, false, reset_count, diag, nullptr, &c));
  std::vector<OsciProblem> ps((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const tj2_osci_tensor& x = tensors[i];
    const tj2_status st = osci_problem(x.W, x.W_prev, nullptr, nullptr, nullptr, x.Q_prev, x.dQ, x.dM, x.N, x.K,
                                       false, x.plan, x.Wq_out, x.W8_out, &ps[(size_t)i]);
    if (st != TJ2_OK) return fail(st, "tensors[%d]: %s", i, std::string(tj2_last_error()).c_str());
  }
  TJ2_TRY(run_osci(c, ps, false, (hipStream_t)stream));
  return ok();
}

size_t tj2_channel_sumsq_workspace_size(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return sumsq_workspace_bytes(M, K);
}

tj2_status tj2_channel_sumsq(const void* X, int64_t M, int64_t K, double* acc, void* workspace, size_t ws_bytes,
                             void* stream) {
  if (!X || !acc || !workspace) return fail(TJ2_ERR_ARG, "X, acc and workspace are required");
  if (!aligned16(X) || !aligned16(acc) || !aligned16(workspace)) return fail(TJ2_ERR_ALIGN, "X, acc and workspace must be 16-byte aligned");
  if (M <= 0 || M > ((int64_t)1 << 30)) return fail(TJ2_ERR_SHAPE, "M must be positive");
  TJ2_TRY(check_dims(K, "K"));
  const size_t need = sumsq_workspace_bytes(M, K);
  if (ws_bytes < need) return fail(TJ2_ERR_ARG, "workspace of %zu bytes required (got %zu)", need, ws_bytes);
  TJ2_TRY(hip_check(launch_channel_sumsq(X, M, K, acc, reinterpret_cast<double*>(workspace), (hipStream_t)stream),
                    "sumsq launch"));
  return ok();
}

tj2_status tj2_select_outliers(const double* scores, int64_t K, double p, int32_t* outliers, int32_t* rest,
                               int32_t* n_outliers) {
  if (!scores || !outliers || !rest || !n_outliers) return fail(TJ2_ERR_ARG, "scores, outliers, rest and n_outliers are required");
  TJ2_TRY(check_dims(K, "K"));
  if (!(p > 0.0 && p < 1.0)) return fail(TJ2_ERR_ARG, "p must lie in (0, 1)");
  for (int64_t k = 0; k < K; ++k)
    if (!(scores[k] >= 0.0) || scores[k] > 1.79e308) return fail(TJ2_ERR_ARG, "score %lld is negative or not finite", (long long)k);
  const int64_t n = (int64_t)ceil(p * (double)K / 16.0) * 16;
  if (n <= 0 || n >= K) return fail(TJ2_ERR_SHAPE, "%lld outlier channels of K = %lld leave no NVFP4 channel", (long long)n, (long long)K);
  std::vector<int32_t> order((size_t)K);
  for (int64_t k = 0; k < K; ++k) order[(size_t)k] = (int32_t)k;
  // descending score, ties to the lower channel index: a strict weak order, so the
  // selection does not depend on the sort's implementation
  std::sort(order.begin(), order.end(), [scores](int32_t a, int32_t b) {
    return scores[a] > scores[b] || (scores[a] == scores[b] && a < b);
  });
  std::vector<uint8_t> is_out((size_t)K, 0);
  for (int64_t i = 0; i < n; ++i) is_out[(size_t)order[(size_t)i]] = 1;
  int64_t no = 0, nr = 0;
  for (int64_t k = 0; k < K; ++k) {
    if (is_out[(size_t)k]) outliers[no++] = (int32_t)k;
    else rest[nr++] = (int32_t)k;
  }
  *n_outliers = (int32_t)n;
  return ok();
}

}  // extern "C"
