// Double-block NVFP4 / per-128 FP8 quantizers for gfx950.
//
// TetraJet-v2 technical summary, section 2.A (double-block quantization:
// 128-element outer blocks with an FP32 scale over 16-element inner blocks with
// an 8-bit scale; round-to-nearest forward, stochastic rounding backward; 1x16
// weight groups whose transpose is re-grouped) and section 2.C (Hadamard
// transform on the backward operands; FP8 outlier channels).
//
// Two kernels, both HBM-bound streaming passes with no global reduction:
//  * quant_row: groups along the contiguous dimension.  One lane owns one
//    16-element group; the 8 lanes of an outer block reduce its amax with DPP.
//  * quant_col: groups along rows, output stored transposed.  One lane owns a
//    16-row x 8-column patch (8 groups, one per column); the 8 lanes stacked
//    along rows form a 128-row outer block.  A row of the patch is one 16-byte
//    (bf16) load, so lanes with neighbouring column patches read contiguous
//    128-byte segments.  Stochastic draws follow the output position, so each
//    16-element group uses two whole Philox blocks generated on the spot.
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

// ----------------------------------------------------------------------------
// Per-group quantization of 16 values v (already transformed if RHT), given
// the outer amax a_o and, for SR, the draws r (top-aligned 16-bit).  Writes 8
// bytes (NVFP4) or 16 bytes (FP8) of codes.
// ----------------------------------------------------------------------------
template <bool FP8OUT, bool SR>
__device__ __forceinline__ void quantize_group(const float v[16], float a_o, float a_j, const uint32_t r[16],
                                               uint32_t codes[4], uint32_t* s_code, float* S_out) {
  if (!FP8OUT) {
    GroupScale g = nvfp4_group_scale(a_o, a_j);
    *s_code = g.s_code;
    *S_out = g.S;
    // both conversions saturate at +-6 and y * 0 keeps the sign of y, so an
    // empty group (inv = 0) encodes signed zeros
    float y[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) y[t] = v[t] * g.inv;
    if (SR) e2m1_sr16(y, r, codes);
    else e2m1_rtn16(y, codes);
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
      codes[0] = codes[1] = codes[2] = codes[3] = 0u;
#pragma unroll
      for (int t = 0; t < 16; ++t) codes[t >> 2] |= e4m3_rne(y[t]) << (8 * (t & 3));
    }
  }
}

// ----------------------------------------------------------------------------
// Row grouping: one lane per 16-element group.
// ----------------------------------------------------------------------------
template <int IN, bool GATHER, bool FP8OUT, bool SR, bool RHT>
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
    const typename Dense<IN>::T* xr = x + (int64_t)row * ld_x;
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
    const uint64_t e0 = (uint64_t)row * (uint64_t)L + j * 16u;
    draws8(e0 >> 3, seed, offset, u);
    draws8((e0 >> 3) + 1, seed, offset, u + 8);
  }
  uint32_t codes[4], s_code;
  float S;
  quantize_group<FP8OUT, SR>(v, a_o, a_j, u, codes, &s_code, &S);

  if (!FP8OUT) {
    *reinterpret_cast<uint2*>(out.codes + (int64_t)row * out.ld_codes + j * 8u) = make_uint2(codes[0], codes[1]);
    out.s16[(int64_t)row * out.ld_s16 + j] = (uint8_t)s_code;
  } else {
    *reinterpret_cast<uint4*>(out.codes + (int64_t)row * out.ld_codes + j * 16u) =
        make_uint4(codes[0], codes[1], codes[2], codes[3]);
  }
  if ((j & 7u) == 0u) out.s128[(int64_t)row * out.ld_s128 + (j >> 3)] = S;
}

// ----------------------------------------------------------------------------
// Column grouping (16x1), output transposed.  Lane (cg, rs) of a wave owns
// columns c0..c0+7 and rows r0..r0+15 of the input; lanes rs = 0..7 of one cg
// are consecutive, so the 128-row outer amax is an 8-lane DPP reduction.
// ----------------------------------------------------------------------------
template <int IN>
struct ColPatch;

template <>
struct ColPatch<TJ2_BF16> {
  uint32_t w[16][4];
  __device__ __forceinline__ void load(const QuantParams& p, int64_t r0, int64_t c0) {
    const uint16_t* x = reinterpret_cast<const uint16_t*>(p.x);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      uint4 a = *reinterpret_cast<const uint4*>(x + (r0 + t) * p.ld_x + c0);
      w[t][0] = a.x; w[t][1] = a.y; w[t][2] = a.z; w[t][3] = a.w;
    }
  }
  __device__ __forceinline__ float get(int t, int k) const {
    uint32_t x = w[t][k >> 1];
    return __uint_as_float((k & 1) ? (x & 0xFFFF0000u) : (x << 16));
  }
};

template <>
struct ColPatch<TJ2_F32> {
  float w[16][8];
  __device__ __forceinline__ void load(const QuantParams& p, int64_t r0, int64_t c0) {
    const float* x = reinterpret_cast<const float*>(p.x);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float4 a = *reinterpret_cast<const float4*>(x + (r0 + t) * p.ld_x + c0);
      float4 b = *reinterpret_cast<const float4*>(x + (r0 + t) * p.ld_x + c0 + 4);
      w[t][0] = a.x; w[t][1] = a.y; w[t][2] = a.z; w[t][3] = a.w;
      w[t][4] = b.x; w[t][5] = b.y; w[t][6] = b.z; w[t][7] = b.w;
    }
  }
  __device__ __forceinline__ float get(int t, int k) const { return w[t][k]; }
};

template <int IN, bool FP8OUT, bool SR, bool RHT>
__global__ __launch_bounds__(256) void quant_col_kernel(QuantParams p) {
  constexpr int CPL = 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cg = lane >> 3, rs = lane & 7;
  const int64_t c0 = ((int64_t)blockIdx.x * 4 + wave) * (8 * CPL) + cg * CPL;
  if (c0 >= p.cols) return;  // all 8 lanes of this column patch exit together
  const int64_t r0 = (int64_t)blockIdx.y * 128 + rs * 16;
  const bool valid = r0 < p.rows;
  const int64_t R = p.rows;

  ColPatch<IN> patch;
  if (valid) patch.load(p, r0, c0);

  const QView& o = p.out;
  static_for<CPL>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    float v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = valid ? patch.get(t, k) : 0.0f;
    if (RHT && valid) rht16(v, p.rht_mask);
    float a_j = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) a_j = fmaxf(a_j, fabsf(v[t]));
    const float a_o = max8_lanes(a_j);
    const int64_t orow = c0 + k;  // output row = input column
    uint32_t u[16];
    if (SR) {  // groups past the last row are zeros: any draw keeps them zero
      // draws follow the output position orow * R + r0 + t: two whole Philox blocks
      const uint64_t b = ((uint64_t)orow * (uint64_t)R + (uint64_t)r0) >> 3;
      draws8(b, p.seed, p.offset, u);
      draws8(b + 1, p.seed, p.offset, u + 8);
    }
    uint32_t codes[4], s_code;
    float S;
    quantize_group<FP8OUT, SR>(v, a_o, a_j, u, codes, &s_code, &S);
    if (!FP8OUT) {
      *reinterpret_cast<uint2*>(o.codes + orow * o.ld_codes + (r0 >> 1)) = make_uint2(codes[0], codes[1]);
      o.s16[orow * o.ld_s16 + (r0 >> 4)] = (uint8_t)s_code;
    } else {
      *reinterpret_cast<uint4*>(o.codes + orow * o.ld_codes + r0) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
    }
    if (rs == 0) o.s128[orow * o.ld_s128 + blockIdx.y] = S;
  });
}

// Packed inputs (NVFP4 / FP8: the forward's operands re-grouped for the
// backward) through LDS: a workgroup stages a 128-row x 64-column tile with
// coalesced row reads, then each lane takes 2 columns x 16 rows of it, as the
// lane layout above (wave w: tile columns 16w..16w+15).
template <int IN>
struct PackedTile;

template <>
struct PackedTile<TJ2_NVFP4> {
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
    if (in) v = *reinterpret_cast<const uint4*>(q.codes + r * q.ld_codes + (c0 >> 1) + half * 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * kRowBytes + half * 16);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    if (half == 0) {
      const uint32_t w = in ? *reinterpret_cast<const uint32_t*>(q.s16 + r * q.ld_s16 + (c0 >> 4)) : 0u;
      *reinterpret_cast<uint32_t*>(s16 + row * 4) = w;
    } else {
      S[row] = in ? q.s128[r * q.ld_s128 + (c0 >> 7)] : 0.0f;
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
struct PackedTile<TJ2_FP8> {
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
      const uint4* src = reinterpret_cast<const uint4*>(q.codes + r * q.ld_codes + c0 + half * 32);
      v0 = src[0];
      v1 = src[1];
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * kRowBytes + half * 32);
    dst[0] = v0.x; dst[1] = v0.y; dst[2] = v0.z; dst[3] = v0.w;
    dst[4] = v1.x; dst[5] = v1.y; dst[6] = v1.z; dst[7] = v1.w;
    if (half == 0) S[row] = in ? q.s128[r * q.ld_s128 + (c0 >> 7)] : 0.0f;
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

template <int IN, bool FP8OUT, bool SR, bool RHT>
__global__ __launch_bounds__(256) void quant_col_packed_kernel(QuantParams p) {
  __shared__ PackedTile<IN> tile;
  const int64_t c_tile = (int64_t)blockIdx.x * 64;
  const int64_t rb = (int64_t)blockIdx.y * 128;
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
      const uint64_t b = ((uint64_t)orow * (uint64_t)R + (uint64_t)r0) >> 3;
      draws8(b, p.seed, p.offset, u);
      draws8(b + 1, p.seed, p.offset, u + 8);
    }
    uint32_t codes[4], s_code;
    float S;
    quantize_group<FP8OUT, SR>(v, a_o, a_j, u, codes, &s_code, &S);
    // groups past the last row are the zero padding of the output's last block
    if (!FP8OUT) {
      *reinterpret_cast<uint2*>(o.codes + orow * o.ld_codes + (r0 >> 1)) = make_uint2(codes[0], codes[1]);
      o.s16[orow * o.ld_s16 + (r0 >> 4)] = (uint8_t)s_code;
    } else {
      *reinterpret_cast<uint4*>(o.codes + orow * o.ld_codes + r0) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
    }
    if (rs == 0) o.s128[orow * o.ld_s128 + blockIdx.y] = S;
  });
}

template <int IN, bool GATHER, bool FP8OUT, bool SR, bool RHT>
hipError_t run_row(const QuantParams& p, hipStream_t s) {
  const int64_t L = p.out.len;
  const int64_t gpr = p.out.nb * 8;
  const int64_t threads = p.rows * gpr;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((quant_row_kernel<IN, GATHER, FP8OUT, SR, RHT>), dim3((uint32_t)blocks), dim3(256), 0, s,
                     reinterpret_cast<const typename Dense<IN>::T*>(p.x), p.ld_x, p.idx, (int32_t)p.rows,
                     (int32_t)L, (int32_t)gpr, p.out, p.rht_mask, p.seed, p.offset);
  return hipGetLastError();
}

template <int IN, bool FP8OUT, bool SR, bool RHT>
hipError_t run_col(const QuantParams& p, hipStream_t s) {
  const int64_t nbR = (p.rows + 127) / 128;
  if constexpr (IN == TJ2_NVFP4 || IN == TJ2_FP8) {
    dim3 grid((uint32_t)((p.cols + 63) / 64), (uint32_t)nbR);
    hipLaunchKernelGGL((quant_col_packed_kernel<IN, FP8OUT, SR, RHT>), grid, dim3(256), 0, s, p);
  } else {
    dim3 grid((uint32_t)((p.cols + 255) / 256), (uint32_t)nbR);
    hipLaunchKernelGGL((quant_col_kernel<IN, FP8OUT, SR, RHT>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <int IN, bool GATHER, bool FP8OUT>
hipError_t dispatch_row_rs(const QuantParams& p, hipStream_t s) {
  const bool sr = p.rounding == TJ2_SR, rht = p.rht != 0;
  if (sr) return rht ? run_row<IN, GATHER, FP8OUT, true, true>(p, s) : run_row<IN, GATHER, FP8OUT, true, false>(p, s);
  return rht ? run_row<IN, GATHER, FP8OUT, false, true>(p, s) : run_row<IN, GATHER, FP8OUT, false, false>(p, s);
}

template <int IN, bool FP8OUT>
hipError_t dispatch_col_rs(const QuantParams& p, hipStream_t s) {
  const bool sr = p.rounding == TJ2_SR, rht = p.rht != 0;
  if (sr) return rht ? run_col<IN, FP8OUT, true, true>(p, s) : run_col<IN, FP8OUT, true, false>(p, s);
  return rht ? run_col<IN, FP8OUT, false, true>(p, s) : run_col<IN, FP8OUT, false, false>(p, s);
}

template <int IN>
hipError_t dispatch_row(const QuantParams& p, hipStream_t s) {
  const bool fp8 = p.out.fmt == TJ2_FP8;
  if (p.idx) return fp8 ? dispatch_row_rs<IN, true, true>(p, s) : dispatch_row_rs<IN, true, false>(p, s);
  return fp8 ? dispatch_row_rs<IN, false, true>(p, s) : dispatch_row_rs<IN, false, false>(p, s);
}

template <int IN>
hipError_t dispatch_col(const QuantParams& p, hipStream_t s) {
  return p.out.fmt == TJ2_FP8 ? dispatch_col_rs<IN, true>(p, s) : dispatch_col_rs<IN, false>(p, s);
}

}  // namespace

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
