// Double-block NVFP4 / per-128 FP8 quantizers for gfx950.
//
// TetraJet-v2 technical summary, section 2.A (double-block quantization:
// 128-element outer blocks with an FP32 scale over 16-element inner blocks with
// an 8-bit scale; round-to-nearest forward, stochastic rounding backward; 1x16
// weight groups whose transpose is re-grouped) and section 2.C (Hadamard
// transform on the backward operands; FP8 outlier channels).
//
// Single-pass kernels with no global reduction (the double block's purpose):
//  * quant_row: groups along the contiguous dimension.  One lane owns one
//    16-element group; the 8 lanes of an outer block reduce its amax with DPP.
//  * quant_col: groups along rows, output stored transposed.  A workgroup
//    stages a 128-row x 64-column input tile in LDS with coalesced row reads;
//    a lane takes two columns x 16 rows (one group per column) and the 8 lanes
//    stacked along rows form a 128-row outer block.  Packed NVFP4 / FP8 inputs
//    (the forward's operands, re-grouped for the backward) are decoded from the
//    tile.  quant_col_multi runs several such problems in one launch.
//  * quant_split: the forward's one read of X (or W) into its NVFP4 rest
//    columns and FP8 outlier columns, whole rows staged in LDS.
// Stochastic draws follow the output position (Philox blocks of 8 elements,
// generated on the spot).  Round-to-nearest passes are bound by HBM; with
// stochastic rounding and the Hadamard transform the arithmetic (Philox,
// butterflies) bounds them.
#include <algorithm>
#include <cstring>

#include "tj2_device.h"
#include "tj2_internal.h"

namespace tj2 {

namespace {

// ----------------------------------------------------------------------------
// loading helpers
// ----------------------------------------------------------------------------
template <int IN>
struct Dense;

template <>
struct Dense<TJ2_BF16> {
  using T = uint16_t;
  // 16 consecutive elements
  static __device__ __forceinline__ void load16(const T* p, float v[16]) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    uint4 a = q[0], b = q[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ float load1(const T* p) { return __uint_as_float((uint32_t)(*p) << 16); }
};

template <>
struct Dense<TJ2_F32> {
  using T = float;
  static __device__ __forceinline__ void load16(const T* p, float v[16]) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 a = q[i];
      v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
    }
  }
  static __device__ __forceinline__ float load1(const T* p) { return *p; }
};

// Butterflies h = 1, 2, 4, 8 of the 16-wide Hadamard transform without its
// final 1/4 (the quantize_group X4 form).
__device__ __forceinline__ void butterflies16(float v[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

// ----------------------------------------------------------------------------
// Per-group quantization of 16 values v (already transformed if RHT), given
// the outer amax a_o and, for SR, the draws r (top-aligned 16-bit).  Writes 8
// bytes (NVFP4) or 16 bytes (FP8, NVFP6) of codes.
//
// X4 (NVFP4 / NVFP6 only): v holds four times the values, the Hadamard
// butterflies of bf16 input without the transform's final 1/4 (a_o and a_j
// are those of the values).  Such sums are multiples of 2^-133, so v / 4 is
// exact and y = (v / 4) * inv is the one rounding of v * inv / 4, which
// v * (inv / 4) also is when inv / 4 is exact (inv >= 2^-124 or 0); otherwise
// (outer amax above about 1e38) v is scaled first.
// ----------------------------------------------------------------------------
template <int OF, bool SR, bool X4 = false>
__device__ __forceinline__ void quantize_group(float v[16], float a_o, float a_j, const uint32_t r[16],
                                               uint32_t codes[4], uint32_t* s_code, float* S_out) {
  if constexpr (OF == TJ2_NVFP4 || OF == TJ2_NVFP6) {
    GroupScale g = OF == TJ2_NVFP4 ? nvfp4_group_scale(a_o, a_j) : nvfp6_group_scale(a_o, a_j);
    *s_code = g.s_code;
    *S_out = g.S;
    if constexpr (X4) {
      if (g.inv >= 0x1p-124f || g.inv == 0.0f) {
        g.inv *= 0.25f;
      } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) v[t] *= 0.25f;
      }
    }
    float y[16];
    if constexpr (OF == TJ2_NVFP4) {
      // both conversions saturate at +-6 and y * 0 keeps the sign of y, so an
      // empty group (inv = 0) encodes signed zeros
#pragma unroll
      for (int t = 0; t < 16; ++t) y[t] = v[t] * g.inv;
      if (SR) e2m1_sr16(y, r, codes);
      else e2m1_rtn16(y, codes);
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) y[t] = fminf(fmaxf(v[t] * g.inv, -7.5f), 7.5f);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t c = 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          c |= (SR ? e2m3_sr_e4m3(y[4 * w + b], r[4 * w + b]) : e2m3_rtn_e4m3(y[4 * w + b])) << (8 * b);
        codes[w] = c;
      }
    }
  } else {
    float S = 0.0f, inv = 0.0f;
    if (a_o >= kTiny) {
      S = a_o / kFp8Div;
      inv = 1.0f / S;
    }
    *s_code = 0u;
    *S_out = S;
    float y[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) y[t] = fp8_scaled(v[t], inv);
    if (SR) {
      e4m3_sr16(y, r, codes);
    } else {
      e4m3_rne16(y, codes);
    }
  }
}

// Codes and scales of one 16-element group of row `row` (group j of the row);
// the entry points bound rows, lengths and strides by 2^30.
template <int OF>
__device__ __forceinline__ void store_group(const QView& o, int64_t row, int64_t j, const uint32_t codes[4],
                                            uint32_t s_code) {
  if constexpr (OF == TJ2_NVFP4) {
    *reinterpret_cast<uint2*>(o.codes + mul32(row, o.ld_codes) + j * 8) = make_uint2(codes[0], codes[1]);
  } else {
    *reinterpret_cast<uint4*>(o.codes + mul32(row, o.ld_codes) + j * 16) =
        make_uint4(codes[0], codes[1], codes[2], codes[3]);
  }
  if constexpr (OF != TJ2_FP8) o.s16[mul32(row, o.ld_s16) + j] = (uint8_t)s_code;
}

// ----------------------------------------------------------------------------
// Row grouping: one lane per 16-element group.
// ----------------------------------------------------------------------------
template <int IN, bool GATHER, int OF, bool SR, bool RHT>
__global__ __launch_bounds__(256) void quant_row_kernel(const typename Dense<IN>::T* __restrict__ x,
                                                        int64_t ld_x, const int32_t* __restrict__ idx,
                                                        int32_t rows, int32_t L, int32_t groups_per_row,
                                                        QView out, uint32_t rht_mask, uint64_t seed,
                                                        uint64_t offset) {
  const uint32_t g = blockIdx.x * 256u + threadIdx.x;
  const uint32_t row = g / (uint32_t)groups_per_row;
  if (row >= (uint32_t)rows) return;  // groups_per_row is a multiple of 8: whole outer blocks exit
  const uint32_t j = g - row * (uint32_t)groups_per_row;
  const bool valid = (int32_t)(j * 16u) < L;

  float v[16];
  if (valid) {
    const typename Dense<IN>::T* xr = x + mul32(row, ld_x);
    if (GATHER) {
      const int4* ip = reinterpret_cast<const int4*>(idx + j * 16u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int4 c = ip[q];
        v[4 * q + 0] = Dense<IN>::load1(xr + c.x);
        v[4 * q + 1] = Dense<IN>::load1(xr + c.y);
        v[4 * q + 2] = Dense<IN>::load1(xr + c.z);
        v[4 * q + 3] = Dense<IN>::load1(xr + c.w);
      }
    } else {
      Dense<IN>::load16(xr + j * 16u, v);
    }
    if (RHT) rht16(v, rht_mask);
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = 0.0f;
  }

  float a_j = 0.0f;
#pragma unroll
  for (int t = 0; t < 16; ++t) a_j = fmaxf(a_j, fabsf(v[t]));
  const float a_o = max8_lanes(a_j);

  // padding groups take draws as well: their values are zero, which every draw
  // rounds to zero, and no branch keeps the draws' registers apart
  uint32_t u[16];
  if (SR) {
    const uint64_t e0 = mul32(row, L) + j * 16u;
    draws8(e0 >> 3, seed, offset, u);
    draws8((e0 >> 3) + 1, seed, offset, u + 8);
  }
  uint32_t codes[4], s_code;
  float S;
  quantize_group<OF, SR>(v, a_o, a_j, u, codes, &s_code, &S);
  store_group<OF>(out, row, j, codes, s_code);
  if ((j & 7u) == 0u) out.s128[mul32(row, out.ld_s128) + (j >> 3)] = S;
}

// ----------------------------------------------------------------------------
// Column grouping (16x1), output transposed.  A workgroup stages a 128-row x
// 64-column tile of the input in LDS with coalesced row reads; lane (cg, rs) of
// wave w then takes tile columns 16w + 2cg, +1 and rows 16rs..16rs+15, one
// 16-element group per column.  Lanes rs = 0..7 of one cg are consecutive, so
// the 128-row outer amax is an 8-lane DPP reduction.  Inputs: bf16 / fp32
// activations and gradients, or the forward's packed NVFP4 / FP8 operands
// (X-hat, W-hat, the FP8 slices) re-grouped for the backward.
// ----------------------------------------------------------------------------
template <int IN>
struct ColTile;

template <>
struct ColTile<TJ2_BF16> {
  static constexpr int kRowWords = 32 + 1;  // 64 bf16, padded
  uint32_t w[128 * kRowWords];
  __device__ __forceinline__ void load(const QuantParams& p, int64_t rb, int64_t c_tile) {
    const uint16_t* x = reinterpret_cast<const uint16_t*>(p.x);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = threadIdx.x + 256 * i, row = idx >> 3, seg = idx & 7;
      const int64_t r = rb + row, c = c_tile + seg * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < p.rows && c < p.cols) v = *reinterpret_cast<const uint4*>(x + mul32(r, p.ld_x) + c);
      uint32_t* d = w + row * kRowWords + seg * 4;
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
  }
  __device__ __forceinline__ void get2(int row, int col, float& v0, float& v1) const {
    const uint32_t b = w[row * kRowWords + (col >> 1)];
    v0 = __uint_as_float(b << 16);
    v1 = __uint_as_float(b & 0xFFFF0000u);
  }
};

template <>
struct ColTile<TJ2_F32> {
  static constexpr int kRowWords = 64 + 2;  // padded, rows stay 8-byte aligned
  float w[128 * kRowWords];
  __device__ __forceinline__ void load(const QuantParams& p, int64_t rb, int64_t c_tile) {
    const float* x = reinterpret_cast<const float*>(p.x);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = threadIdx.x + 256 * i, row = idx >> 4, seg = idx & 15;
      const int64_t r = rb + row, c = c_tile + seg * 4;
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (r < p.rows && c < p.cols) v = *reinterpret_cast<const float4*>(x + mul32(r, p.ld_x) + c);
      float* d = w + row * kRowWords + seg * 4;
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
  }
  __device__ __forceinline__ void get2(int row, int col, float& v0, float& v1) const {
    const float2 b = *reinterpret_cast<const float2*>(w + row * kRowWords + col);
    v0 = b.x;
    v1 = b.y;
  }
};

template <>
struct ColTile<TJ2_NVFP4> {
  static constexpr int kRowBytes = 32 + 4;  // codes of 64 columns, padded
  uint8_t codes[128 * kRowBytes];
  uint8_t s16[128 * 4];
  float S[128];
  __device__ __forceinline__ void load(const QuantParams& p, int64_t rb, int64_t c0) {
    const QView& q = p.xq;
    const int t = threadIdx.x, row = t >> 1, half = t & 1;
    const int64_t r = rb + row;
    const bool in = r < p.rows;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (in) v = *reinterpret_cast<const uint4*>(q.codes + mul32(r, q.ld_codes) + (c0 >> 1) + half * 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * kRowBytes + half * 16);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    if (half == 0) {
      const uint32_t w = in ? *reinterpret_cast<const uint32_t*>(q.s16 + mul32(r, q.ld_s16) + (c0 >> 4)) : 0u;
      *reinterpret_cast<uint32_t*>(s16 + row * 4) = w;
    } else {
      S[row] = in ? q.s128[mul32(r, q.ld_s128) + (c0 >> 7)] : 0.0f;
    }
  }
  // values of tile row `row`, tile columns col, col + 1 (col even): (q * s) * S in fp32,
  // the forward's X-hat / W-hat
  __device__ __forceinline__ void get2(int row, int col, float& v0, float& v1) const {
    typedef float float2_t __attribute__((ext_vector_type(2)));
    const uint32_t b = codes[row * kRowBytes + (col >> 1)];
    const float s = e4m3_decode(s16[row * 4 + (col >> 4)]);
    const float Sr = S[row];
    const float2_t q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b, 1.0f, 0);  // exact E2M1 values
    v0 = (q.x * s) * Sr;
    v1 = (q.y * s) * Sr;
  }
};

template <>
struct ColTile<TJ2_FP8> {
  static constexpr int kRowBytes = 64 + 4;
  uint8_t codes[128 * kRowBytes];
  float S[128];
  __device__ __forceinline__ void load(const QuantParams& p, int64_t rb, int64_t c0) {
    const QView& q = p.xq;
    const int t = threadIdx.x, row = t >> 1, half = t & 1;
    const int64_t r = rb + row;
    const bool in = r < p.rows;
    uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = v0;
    if (in) {
      const uint4* src = reinterpret_cast<const uint4*>(q.codes + mul32(r, q.ld_codes) + c0 + half * 32);
      v0 = src[0];
      v1 = src[1];
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * kRowBytes + half * 32);
    dst[0] = v0.x; dst[1] = v0.y; dst[2] = v0.z; dst[3] = v0.w;
    dst[4] = v1.x; dst[5] = v1.y; dst[6] = v1.z; dst[7] = v1.w;
    if (half == 0) S[row] = in ? q.s128[mul32(r, q.ld_s128) + (c0 >> 7)] : 0.0f;
  }
  __device__ __forceinline__ void get2(int row, int col, float& v0, float& v1) const {
    typedef float float2_t __attribute__((ext_vector_type(2)));
    const uint32_t b = *reinterpret_cast<const uint16_t*>(codes + row * kRowBytes + col);
    const float Sr = S[row];
    const float2_t q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b, 1.0f, false);  // exact E4M3 values
    v0 = q.x * Sr;
    v1 = q.y * Sr;
  }
};

// The image of a product's B operand (its f16 decode, laid out as the
// product's LDS stage; see kImgRowBytes): this group's 16 values, decoded
// exactly as the product would (E2M1 times its E4M3 scale, or the E4M3 value;
// the outer scale S stays a separate float), go to image row img_rows[orow]
// (or orow), chunk g, elements 16 rs .. 16 rs + 15; lane rs = 0 writes S.
template <int OF>
__device__ __forceinline__ void write_image_group(uint8_t* img, float* img_sc, int64_t img_ld, int64_t img_nch,
                                                  int64_t d, uint32_t g, int rs, const uint32_t codes[4],
                                                  uint32_t s_code, float S) {
  uint8_t* dst = img + (mul32(d >> 7, img_nch) + g) * kImgChunkBytes + (size_t)(d & 127) * kImgRowBytes + rs * 32;
  uint32_t h[8];
  if constexpr (OF == TJ2_NVFP4) {
    const half2_t s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s_code, 1.0f, false);
    const half2_t sc = half2_t{s2[0], s2[0]};
    static_for<8>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      const half2_t q = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[i >> 2], 1.0f, i & 3) * sc;
      h[i] = __builtin_bit_cast(uint32_t, q);
    });
  } else {
    static_for<8>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      h[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[i >> 1], 1.0f, (i & 1) != 0));
    });
  }
  *reinterpret_cast<uint4*>(dst) = make_uint4(h[0], h[1], h[2], h[3]);
  *reinterpret_cast<uint4*>(dst + 16) = make_uint4(h[4], h[5], h[6], h[7]);
  if (rs == 0) img_sc[mul32(g, img_ld) + (size_t)d] = S;
}

template <int OF>
__device__ __forceinline__ void store_image_group(const QuantParams& p, int64_t orow, uint32_t g, int rs,
                                                  const uint32_t codes[4], uint32_t s_code, float S) {
  const int64_t d = p.img_rows ? (int64_t)p.img_rows[orow] : orow;
  write_image_group<OF>(p.img, p.img_sc, p.img_ld, p.img_nch, d, g, rs, codes, s_code, S);
}

// One 128-row x 64-column tile (number `bid` of the problem's tiles).
template <int IN, int OF, bool SR, bool RHT>
__device__ __forceinline__ void col_tile(const QuantParams& p, uint32_t bid, ColTile<IN>& tile) {
  // Packed inputs: row blocks fastest, so the column tiles of one row block run
  // on one XCD (and its L2) close together and a cache line holding several of
  // their packed rows is fetched from HBM once.  Dense inputs: column tiles
  // fastest (a tile row is a whole 128-byte line; neighbours share DRAM pages).
  constexpr bool kRowsFastest = IN == TJ2_NVFP4 || IN == TJ2_FP8;
  const uint32_t nbR = (uint32_t)((p.rows + 127) / 128);
  const uint32_t nbC = (uint32_t)((p.cols + 63) / 64);
  const uint32_t rbi = kRowsFastest ? bid % nbR : bid / nbC;
  const uint32_t cti = kRowsFastest ? bid / nbR : bid % nbC;
  const int64_t c_tile = (int64_t)cti * 64;
  const int64_t rb = (int64_t)rbi * 128;
  tile.load(p, rb, c_tile);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cg = lane >> 3, rs = lane & 7;
  const int cl = wave * 16 + cg * 2;  // first of this lane's two tile columns
  const int64_t c0 = c_tile + cl;
  if (c0 >= p.cols) return;  // all 8 lanes of this column pair exit together
  const int64_t r0 = rb + rs * 16;
  const bool valid = r0 < p.rows;
  const int64_t R = p.rows;
  const QView& o = p.out;
  float vv[2][16];
#pragma unroll
  for (int t = 0; t < 16; ++t) tile.get2(rs * 16 + t, cl, vv[0][t], vv[1][t]);
  static_for<2>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    float* v = vv[k];
    if (RHT && valid) rht16(v, p.rht_mask);
    float a_j = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) a_j = fmaxf(a_j, fabsf(v[t]));
    const float a_o = max8_lanes(a_j);
    const int64_t orow = c0 + k;  // output row = input column
    uint32_t u[16];
    if (SR) {  // groups past the last row are zeros: any draw keeps them zero
      const uint64_t b = (mul32(orow, R) + (uint64_t)r0) >> 3;
      draws8(b, p.seed, p.offset, u);
      draws8(b + 1, p.seed, p.offset, u + 8);
    }
    uint32_t codes[4], s_code;
    float S;
    quantize_group<OF, SR>(v, a_o, a_j, u, codes, &s_code, &S);
    // groups past the last row are the zero padding of the output's last block
    store_group<OF>(o, orow, r0 >> 4, codes, s_code);
    if (rs == 0) o.s128[mul32(orow, o.ld_s128) + rbi] = S;
    if constexpr (OF == TJ2_NVFP4 || OF == TJ2_FP8) {
      if (p.img) store_image_group<OF>(p, orow, rbi, rs, codes, s_code, S);
    }
  });
}

template <int IN, int OF, bool SR, bool RHT>
__global__ __launch_bounds__(256) void quant_col_kernel(QuantParams p) {
  __shared__ ColTile<IN> tile;
  col_tile<IN, OF, SR, RHT>(p, blockIdx.x, tile);
}

// Several independent column quantizations in one launch (the backward's
// re-grouped operands): workgroups [begin[i], begin[i+1]) take problem i, so
// small, latency-bound problems run beside the large ones instead of after
// them.  Combinations: bf16 -> NVFP4 or NVFP6, NVFP4 -> NVFP4, FP8 -> FP8.
struct ColMulti {
  QuantParams p[kColMultiMax];
  uint32_t begin[kColMultiMax + 1];
  int n;
};
static_assert(sizeof(ColMulti) <= 4096, "kernel arguments stay within 4 KB");

template <bool SR, bool RHT>
__global__ __launch_bounds__(256) void quant_col_multi_kernel(ColMulti m) {
  __shared__ union {
    ColTile<TJ2_BF16> b;
    ColTile<TJ2_NVFP4> n;
    ColTile<TJ2_FP8> e;
  } tile;
  int i = 0;
  while (i + 1 < m.n && blockIdx.x >= m.begin[i + 1]) ++i;  // uniform per workgroup
  const QuantParams& p = m.p[i];
  const uint32_t bid = blockIdx.x - m.begin[i];
  if (p.in_dtype == TJ2_BF16) {
    if (p.out.fmt == TJ2_NVFP6) col_tile<TJ2_BF16, TJ2_NVFP6, SR, RHT>(p, bid, tile.b);
    else col_tile<TJ2_BF16, TJ2_NVFP4, SR, RHT>(p, bid, tile.b);
  } else if (p.in_dtype == TJ2_NVFP4) {
    col_tile<TJ2_NVFP4, TJ2_NVFP4, SR, RHT>(p, bid, tile.n);
  } else {
    col_tile<TJ2_FP8, TJ2_FP8, SR, RHT>(p, bid, tile.e);
  }
}

template <int IN, bool GATHER, int OF, bool SR, bool RHT>
hipError_t run_row(const QuantParams& p, hipStream_t s) {
  const int64_t L = p.out.len;
  const int64_t gpr = p.out.nb * 8;
  const int64_t threads = p.rows * gpr;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((quant_row_kernel<IN, GATHER, OF, SR, RHT>), dim3((uint32_t)blocks), dim3(256), 0, s,
                     reinterpret_cast<const typename Dense<IN>::T*>(p.x), p.ld_x, p.idx, (int32_t)p.rows,
                     (int32_t)L, (int32_t)gpr, p.out, p.rht_mask, p.seed, p.offset);
  return hipGetLastError();
}

template <int IN, int OF, bool SR, bool RHT>
hipError_t run_col(const QuantParams& p, hipStream_t s) {
  const int64_t blocks = (p.cols + 63) / 64 * ((p.rows + 127) / 128);
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((quant_col_kernel<IN, OF, SR, RHT>), dim3((uint32_t)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int IN, bool GATHER, int OF>
hipError_t dispatch_row_rs(const QuantParams& p, hipStream_t s) {
  const bool sr = p.rounding == TJ2_SR, rht = p.rht != 0;
  if (sr) return rht ? run_row<IN, GATHER, OF, true, true>(p, s) : run_row<IN, GATHER, OF, true, false>(p, s);
  return rht ? run_row<IN, GATHER, OF, false, true>(p, s) : run_row<IN, GATHER, OF, false, false>(p, s);
}

template <int IN, int OF>
hipError_t dispatch_col_rs(const QuantParams& p, hipStream_t s) {
  const bool sr = p.rounding == TJ2_SR, rht = p.rht != 0;
  if (sr) return rht ? run_col<IN, OF, true, true>(p, s) : run_col<IN, OF, true, false>(p, s);
  return rht ? run_col<IN, OF, false, true>(p, s) : run_col<IN, OF, false, false>(p, s);
}

template <int IN>
hipError_t dispatch_row(const QuantParams& p, hipStream_t s) {
  const int of = p.out.fmt;
  if (p.idx) return of == TJ2_FP8 ? dispatch_row_rs<IN, true, TJ2_FP8>(p, s) : dispatch_row_rs<IN, true, TJ2_NVFP4>(p, s);
  if (of == TJ2_NVFP6) return dispatch_row_rs<IN, false, TJ2_NVFP6>(p, s);
  return of == TJ2_FP8 ? dispatch_row_rs<IN, false, TJ2_FP8>(p, s) : dispatch_row_rs<IN, false, TJ2_NVFP4>(p, s);
}

template <int IN>
hipError_t dispatch_col(const QuantParams& p, hipStream_t s) {
  if constexpr (IN == TJ2_BF16 || IN == TJ2_F32) {
    if (p.out.fmt == TJ2_NVFP6) return dispatch_col_rs<IN, TJ2_NVFP6>(p, s);
  }
  return p.out.fmt == TJ2_FP8 ? dispatch_col_rs<IN, TJ2_FP8>(p, s) : dispatch_col_rs<IN, TJ2_NVFP4>(p, s);
}

// ----------------------------------------------------------------------------
// Both backward groupings of the output gradient from one read (TetraJet-v2
// technical summary, sections 2.A and 2.C: dY enters dX = Q(dY) Q(W^T) grouped
// along N and dW = Q(dY^T) Q(X^T) grouped along M, each with its own Hadamard
// signs and draws).  A workgroup of 512 lanes stages a 128 x 128 tile of dY (rows m,
// columns n) in LDS with coalesced reads.  Its rows are 8 row groups each, one
// outer block along N, quantized as quant_row does (one lane per group, the 8
// lanes of an outer block consecutive); its columns are 8 column groups each,
// one outer block along M, quantized as quant_col does (a lane takes two
// columns x 16 rows).  Codes, scales and draws equal those of the two separate
// passes.
// ----------------------------------------------------------------------------
// 512 lanes: two row groups and two column groups per lane; 70 VGPRs and 33 KB
// of LDS allow six waves per SIMD (256 lanes: four, 4-8% slower).
constexpr int kDualThreads = 512;
template <int OF, bool RHT>
__global__ __launch_bounds__(kDualThreads) void quant_dual_kernel(DualParams p) {
  constexpr int kT = kDualThreads;
  constexpr int kW = 64 + 1;  // a tile row: 128 bf16 as 64 words, padded
  __shared__ uint32_t tile[128 * kW];
  const uint32_t nbC = (uint32_t)((p.cols + 127) / 128);
  const int64_t rb = (int64_t)(blockIdx.x / nbC) * 128, cb = (int64_t)(blockIdx.x % nbC) * 128;
  {
    // 128 rows x 16 pieces of 16 bytes, all of a lane's in flight before the LDS writes
    uint4 t[2048 / kT];
    const int64_t r0 = rb + (threadIdx.x >> 4), c = cb + (threadIdx.x & 15) * 8;
    const uint16_t* x0 = p.x + mul32(r0, p.cols) + c;
#pragma unroll
    for (int i = 0; i < 2048 / kT; ++i) {
      // pass i: rows r0 + (kT / 16) i
      t[i] = (r0 + (kT / 16) * i < p.rows && c < p.cols)
                 ? *reinterpret_cast<const uint4*>(x0 + (int64_t)(kT / 16) * i * p.cols)
                 : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < 2048 / kT; ++i) {
      const int idx = (int)threadIdx.x + kT * i, row = idx >> 4, seg = idx & 15;
      uint32_t* d = tile + row * kW + seg * 4;
      d[0] = t[i].x; d[1] = t[i].y; d[2] = t[i].z; d[3] = t[i].w;
    }
  }
  __syncthreads();

  // row groups: 1024 per tile
#pragma unroll 1
  for (int pass = 0; pass < 1024 / kT; ++pass) {
    const int g = pass * kT + (int)threadIdx.x, row = g >> 3, j = g & 7;
    const int64_t R = rb + row;
    if (R < p.rows) {  // the 8 lanes of a row exit together
      const bool valid = cb + j * 16 < p.cols;
      float v[16];
      const uint32_t* w = tile + row * kW + j * 8;
      if (RHT && valid) {
        // bf16 -> fp32 with the transform's sign in one instruction per element
        // (a shift-add, where adding 2^31 flips bit 31 only, or an and-xor), then
        // the butterflies
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t b = w[i];
          v[2 * i] = __uint_as_float((b << 16) + rht_sign(p.row_mask, 2 * i));
          v[2 * i + 1] = __uint_as_float((b & 0xFFFF0000u) ^ rht_sign(p.row_mask, 2 * i + 1));
        }
        butterflies16(v);  // four times the transformed values (zeros stay zeros)
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t b = valid ? w[i] : 0u;
          v[2 * i] = __uint_as_float(b << 16);
          v[2 * i + 1] = __uint_as_float(b & 0xFFFF0000u);
        }
      }
      float a_j = 0.0f;
#pragma unroll
      for (int t = 0; t < 16; ++t) a_j = fmaxf(a_j, fabsf(v[t]));
      if (RHT) a_j *= 0.25f;  // exact: the amax of the transformed values
      const float a_o = max8_lanes(a_j);
      uint32_t u[16];
      const uint64_t e0 = mul32(R, p.cols) + (uint64_t)(cb + j * 16);
      draws8(e0 >> 3, p.seed, p.row_offset, u);
      draws8((e0 >> 3) + 1, p.seed, p.row_offset, u + 8);
      uint32_t codes[4], s_code;
      float S;
      quantize_group<OF, true, RHT>(v, a_o, a_j, u, codes, &s_code, &S);
      store_group<OF>(p.row_out, R, (cb >> 4) + j, codes, s_code);
      if (j == 0) p.row_out.s128[mul32(R, p.row_out.ld_s128) + (cb >> 7)] = S;
    }
  }

  // column groups: lane (cg, rs) of wave w takes tile columns 16 (kT / 64) pass + 16w + 2cg, +1
  // and rows 16rs..16rs+15
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cg = lane >> 3, rs = lane & 7;
#pragma unroll 1
  for (int pass = 0; pass < 128 * 64 / (16 * kT); ++pass) {
    const int cl = pass * (kT / 4) + wave * 16 + cg * 2;
    const int64_t c0 = cb + cl;
    if (c0 >= p.cols) continue;  // all 8 lanes of this column pair together
    const int64_t r0 = rb + rs * 16;
    const bool valid = r0 < p.rows;
    float vv[2][16];
    if (RHT && valid) {
      // as the row groups: the sign of row t in the bf16 -> fp32 step
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const uint32_t b = tile[(rs * 16 + t) * kW + (cl >> 1)];
        vv[0][t] = __uint_as_float((b << 16) + rht_sign(p.col_mask, t));
        vv[1][t] = __uint_as_float((b & 0xFFFF0000u) ^ rht_sign(p.col_mask, t));
      }
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const uint32_t b = tile[(rs * 16 + t) * kW + (cl >> 1)];
        vv[0][t] = __uint_as_float(b << 16);
        vv[1][t] = __uint_as_float(b & 0xFFFF0000u);
      }
    }
    static_for<2>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      float* v = vv[k];
      if (RHT && valid) butterflies16(v);  // four times the transformed values
      float a_j = 0.0f;
#pragma unroll
      for (int t = 0; t < 16; ++t) a_j = fmaxf(a_j, fabsf(v[t]));
      if (RHT) a_j *= 0.25f;
      const float a_o = max8_lanes(a_j);
      const int64_t orow = c0 + k;  // output row = input column
      uint32_t u[16];
      const uint64_t b = (mul32(orow, p.rows) + (uint64_t)r0) >> 3;
      draws8(b, p.seed, p.col_offset, u);
      draws8(b + 1, p.seed, p.col_offset, u + 8);
      uint32_t codes[4], s_code;
      float S;
      quantize_group<OF, true, RHT>(v, a_o, a_j, u, codes, &s_code, &S);
      // groups past the last row are the zero padding of the output's last block
      store_group<OF>(p.col_out, orow, r0 >> 4, codes, s_code);
      if (rs == 0) p.col_out.s128[mul32(orow, p.col_out.ld_s128) + (rb >> 7)] = S;
    });
  }
}

}  // namespace

hipError_t launch_quant_dual(const DualParams& p, hipStream_t s) {
  const int64_t tiles = ((p.rows + 127) / 128) * ((p.cols + 127) / 128);
  if (tiles >= ((int64_t)1 << 31) || (p.cols % 16) != 0) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)tiles);
  if (p.row_out.fmt == TJ2_NVFP6) {
    if (p.rht) hipLaunchKernelGGL((quant_dual_kernel<TJ2_NVFP6, true>), grid, dim3(kDualThreads), 0, s, p);
    else hipLaunchKernelGGL((quant_dual_kernel<TJ2_NVFP6, false>), grid, dim3(kDualThreads), 0, s, p);
  } else {
    if (p.rht) hipLaunchKernelGGL((quant_dual_kernel<TJ2_NVFP4, true>), grid, dim3(kDualThreads), 0, s, p);
    else hipLaunchKernelGGL((quant_dual_kernel<TJ2_NVFP4, false>), grid, dim3(kDualThreads), 0, s, p);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Forward split with an outlier plan (TetraJet-v2 technical summary, section
// 2.C): a workgroup stages R whole input rows in LDS with coalesced reads, then
// each lane takes 16-element groups (8 nb(rest) NVFP4 and 8 nb(outl) FP8 ones
// per row) and gathers their columns from LDS.  Groups of one outer block are 8
// consecutive lanes, as in the row kernel, so their amax is a DPP reduction.
// ----------------------------------------------------------------------------
extern __shared__ uint32_t rows_lds[];

// Workgroup blk of a split quantization (rows R * blk ..).
template <int IN>
__device__ __forceinline__ void split_body(const SplitParams& p, int R, uint32_t blk) {
  using T = typename Dense<IN>::T;
  const int64_t r_base = (int64_t)blk * R;
  const int nrows = (int)min((int64_t)R, p.rows - r_base);
  const int units = (int)(p.cols * (int64_t)sizeof(T) / 16);  // 16-byte units per row
  {
    // the rows are contiguous and hold at most 32 KB: eight 16-byte loads per
    // lane, all in flight before the LDS writes
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(p.x) + mul32(r_base, p.cols));
    uint4* dst = reinterpret_cast<uint4*>(rows_lds);
    const int n = nrows * units;
    uint4 t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = i * 256 + (int)threadIdx.x;
      t[i] = u < n ? src[u] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = i * 256 + (int)threadIdx.x;
      if (u < n) dst[u] = t[i];
    }
  }
  __syncthreads();
  const T* xs = reinterpret_cast<const T*>(rows_lds);
  // the NVFP4 groups of all rows first, then the FP8 groups, so that only one
  // wave holds both kinds
  const int G4 = (int)p.q4.nb * 8, G8 = (int)p.q8.nb * 8;
  const int total4 = nrows * G4, total = total4 + nrows * G8;  // multiples of 8
  for (int g = threadIdx.x; g < total; g += 256) {
    const bool fp8 = g >= total4;
    const int Gk = fp8 ? G8 : G4, gk = fp8 ? g - total4 : g;
    const int row = gk / Gk, jj = gk - row * Gk;
    const int64_t len = fp8 ? p.q8.len : p.q4.len;
    const int32_t* idx = fp8 ? p.outl : p.rest;
    const bool valid = (int64_t)jj * 16 < len;
    float v[16];
    if (valid) {
      const int4* ip = reinterpret_cast<const int4*>(idx + jj * 16);
      const T* xr = xs + mul32(row, p.cols);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int4 c = ip[q];
        v[4 * q + 0] = Dense<IN>::load1(xr + c.x);
        v[4 * q + 1] = Dense<IN>::load1(xr + c.y);
        v[4 * q + 2] = Dense<IN>::load1(xr + c.z);
        v[4 * q + 3] = Dense<IN>::load1(xr + c.w);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) v[t] = 0.0f;
    }
    float a_j = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) a_j = fmaxf(a_j, fabsf(v[t]));
    const float a_o = max8_lanes(a_j);
    const int64_t orow = r_base + row;
    uint32_t codes[4], s_code;
    float S;
    if (!fp8) {
      quantize_group<TJ2_NVFP4, false>(v, a_o, a_j, nullptr, codes, &s_code, &S);
      const QView& o = p.q4;
      *reinterpret_cast<uint2*>(o.codes + mul32(orow, o.ld_codes) + jj * 8) = make_uint2(codes[0], codes[1]);
      o.s16[mul32(orow, o.ld_s16) + jj] = (uint8_t)s_code;
      if ((jj & 7) == 0) o.s128[mul32(orow, o.ld_s128) + (jj >> 3)] = S;
      if (p.img)
        write_image_group<TJ2_NVFP4>(p.img, p.img_sc, p.img_ld, p.img_nch, orow, (uint32_t)(jj >> 3), jj & 7, codes,
                                     s_code, S);
    } else {
      quantize_group<TJ2_FP8, false>(v, a_o, a_j, nullptr, codes, &s_code, &S);
      const QView& o = p.q8;
      *reinterpret_cast<uint4*>(o.codes + mul32(orow, o.ld_codes) + jj * 16) =
          make_uint4(codes[0], codes[1], codes[2], codes[3]);
      if ((jj & 7) == 0) o.s128[mul32(orow, o.ld_s128) + (jj >> 3)] = S;
      if (p.img)
        write_image_group<TJ2_FP8>(p.img, p.img_sc, p.img_ld, p.img_nch, orow, (uint32_t)(p.img_g8 + (jj >> 3)),
                                   jj & 7, codes, s_code, S);
    }
  }
}

template <int IN>
__global__ __launch_bounds__(256) void quant_split_kernel(SplitParams p, int R) {
  split_body<IN>(p, R, blockIdx.x);
}

// The forward's two split quantizations in one launch: workgroups [0, bx)
// take X (bf16), the others the fp32 masters W, so the smaller launch's ramp
// and tail overlap the larger one's.
__global__ __launch_bounds__(256) void quant_split2_kernel(SplitParams px, int rx, uint32_t bx, SplitParams pw,
                                                           int rw) {
  if (blockIdx.x < bx) split_body<TJ2_BF16>(px, rx, blockIdx.x);
  else split_body<TJ2_F32>(pw, rw, blockIdx.x - bx);
}


// Rows per workgroup: the groups of R rows fill whole 256-lane passes as well
// as possible, within 32 KB of LDS (several workgroups per CU).
int split_rows_per_wg(int64_t cols, int esize, int64_t groups_per_row) {
  const int64_t rmax = std::max<int64_t>(1, std::min<int64_t>(16, 32768 / (cols * esize)));
  int best = 1;
  double best_eff = 0.0;
  for (int64_t r = 1; r <= rmax; ++r) {
    const int64_t work = r * groups_per_row, passes = (work + 255) / 256;
    const double eff = (double)work / (double)(passes * 256);
    if (eff > best_eff + 1e-9) { best_eff = eff; best = (int)r; }
  }
  return best;
}

hipError_t launch_quant_split2(const SplitParams& px, const SplitParams& pw, hipStream_t s) {
  if (px.in_dtype != TJ2_BF16 || pw.in_dtype != TJ2_F32 || px.cols * 2 > 32768 || pw.cols * 4 > 32768)
    return hipErrorInvalidValue;  // the kernel stages at most 32 KB per workgroup
  const int rx = split_rows_per_wg(px.cols, 2, (px.q4.nb + px.q8.nb) * 8);
  const int rw = split_rows_per_wg(pw.cols, 4, (pw.q4.nb + pw.q8.nb) * 8);
  const uint32_t bx = (uint32_t)((px.rows + rx - 1) / rx), bw = (uint32_t)((pw.rows + rw - 1) / rw);
  const size_t lds = std::max((size_t)rx * px.cols * 2, (size_t)rw * pw.cols * 4);
  hipLaunchKernelGGL(quant_split2_kernel, dim3(bx + bw), dim3(256), lds, s, px, rx, bx, pw, rw);
  return hipGetLastError();
}

hipError_t launch_quant_split(const SplitParams& p, hipStream_t s) {
  const int esize = p.in_dtype == TJ2_BF16 ? 2 : 4;
  if (p.cols * esize > 32768) return hipErrorInvalidValue;  // the kernel stages at most 32 KB
  const int R = split_rows_per_wg(p.cols, esize, (p.q4.nb + p.q8.nb) * 8);
  const uint32_t blocks = (uint32_t)((p.rows + R - 1) / R);
  const size_t lds = (size_t)R * p.cols * esize;
  if (p.in_dtype == TJ2_BF16)
    hipLaunchKernelGGL(quant_split_kernel<TJ2_BF16>, dim3(blocks), dim3(256), lds, s, p, R);
  else
    hipLaunchKernelGGL(quant_split_kernel<TJ2_F32>, dim3(blocks), dim3(256), lds, s, p, R);
  return hipGetLastError();
}

hipError_t launch_quant_col_multi(const QuantParams* ps, int n, hipStream_t s) {
  if (n < 1 || n > kColMultiMax) return hipErrorInvalidValue;
  ColMulti m;
  memset(&m, 0, sizeof(m));
  m.n = n;
  int64_t total = 0;
  bool sr = ps[0].rounding == TJ2_SR, rht = ps[0].rht != 0;
  for (int i = 0; i < n; ++i) {
    const QuantParams& p = ps[i];
    const bool ok = p.grouping == TJ2_GROUP_COL && (p.rounding == TJ2_SR) == sr && (p.rht != 0) == rht &&
                    ((p.in_dtype == TJ2_BF16 && (p.out.fmt == TJ2_NVFP4 || p.out.fmt == TJ2_NVFP6)) ||
                     (p.in_dtype == TJ2_NVFP4 && p.out.fmt == TJ2_NVFP4) ||
                     (p.in_dtype == TJ2_FP8 && p.out.fmt == TJ2_FP8));
    if (!ok) return hipErrorInvalidValue;
    m.p[i] = p;
    m.begin[i] = (uint32_t)total;
    total += (p.cols + 63) / 64 * ((p.rows + 127) / 128);
  }
  if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  m.begin[n] = (uint32_t)total;
  const dim3 grid((uint32_t)total);
  if (sr) {
    if (rht) hipLaunchKernelGGL((quant_col_multi_kernel<true, true>), grid, dim3(256), 0, s, m);
    else hipLaunchKernelGGL((quant_col_multi_kernel<true, false>), grid, dim3(256), 0, s, m);
  } else {
    if (rht) hipLaunchKernelGGL((quant_col_multi_kernel<false, true>), grid, dim3(256), 0, s, m);
    else hipLaunchKernelGGL((quant_col_multi_kernel<false, false>), grid, dim3(256), 0, s, m);
  }
  return hipGetLastError();
}

hipError_t launch_quant(const QuantParams& p, hipStream_t s) {
  if (p.grouping == TJ2_GROUP_ROW) {
    switch (p.in_dtype) {
      case TJ2_BF16: return dispatch_row<TJ2_BF16>(p, s);
      case TJ2_F32: return dispatch_row<TJ2_F32>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.in_dtype) {
    case TJ2_BF16: return dispatch_col<TJ2_BF16>(p, s);
    case TJ2_F32: return dispatch_col<TJ2_F32>(p, s);
    case TJ2_NVFP4: return dispatch_col<TJ2_NVFP4>(p, s);
    case TJ2_FP8: return dispatch_col<TJ2_FP8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tj2
