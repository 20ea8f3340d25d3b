// Products on packed NVFP4 / FP8 operands for gfx950.
//
// TetraJet-v2 technical summary, section 2: activations, weights and gradients
// of every linear layer are NVFP4, so Y = X W^T, dX and dW all run on the
// quantized operands (section 2.C adds FP8 segments for outlier channels).
//
// C[i, j] = sum over 128-element outer blocks kb of  S_A[i,kb] * S_B[j,kb] *
//           sum_{k in kb} (q_A s_A)[i,k] * (q_B s_B)[j,k]
//
// Decode path: an E2M1 value times its E4M3 inner scale needs at most 6
// significant bits and lies in [2^-10, 2688], so it is exact in f16; the FP32
// outer scales cannot be folded into the elements without rounding, so each
// 128-wide K chunk is reduced on MFMA into a fresh f32 partial and promoted
// into the accumulator with one multiply-add by S_A * S_B.  CDNA4's
// block-scaled MFMA takes E8M0 scales per 32 elements, which cannot express an
// E4M3 scale per 16, hence the f16 decode.
//
// Kernel: 128x128 output tile per 256-thread workgroup (2x2 waves of 64x64,
// each 2x2 v_mfma_f32_32x32x16_f16).  Per 128-K chunk every thread loads one
// row-half of A and of B (packed codes + scales), decodes it to f16 with
// v_cvt_scalef32_pk_f16_fp4 / _fp8 (scale 1.0: exact) and v_pk_mul_f16 by the
// inner scale, and writes it to LDS (rows padded to 272 bytes: conflict-free
// 16-byte accesses).  The next chunk's packed operands are fetched into
// registers while the current chunk runs on MFMA; two workgroups per CU
// overlap one's decode with the other's MFMA.
#include "tj2_device.h"
#include "tj2_internal.h"

namespace tj2 {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_STRIDE = BK + 8;  // f16 elements per LDS row

struct OperandK {
  const uint8_t* codes;
  const uint8_t* s16;
  const float* s128;
  int64_t ld_codes, ld_s16, ld_s128;
  int fmt;
};

struct SegK {
  OperandK a, b;
  int64_t K;
  int nchunks;
};

struct GemmKArgs {
  SegK seg[2];
  int nseg;
  int nchunks;
  int64_t I, J;
  void* C;
  int64_t ldc;
  const int32_t* col_map;
  int c_bf16;
  int accumulate;
};

// Packed operand slice of one thread: 64 consecutive K elements of one row.
struct Slice {
  uint4 c[4];      // NVFP4 uses c[0..1] (32 bytes), FP8 c[0..3] (64 bytes)
  uint32_t s16;    // four E4M3 inner scales (NVFP4)
  float S;         // outer scale of the chunk
};

__device__ __forceinline__ void load_slice(const OperandK& o, int64_t row, bool valid, int kc, int half,
                                           Slice& s) {
  if (!valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s.c[i] = make_uint4(0, 0, 0, 0);
    s.s16 = 0u;
    s.S = 0.0f;
    return;
  }
  if (o.fmt == TJ2_NVFP4) {
    const uint4* p = reinterpret_cast<const uint4*>(o.codes + row * o.ld_codes + kc * 64 + half * 32);
    s.c[0] = p[0];
    s.c[1] = p[1];
    s.s16 = *reinterpret_cast<const uint32_t*>(o.s16 + row * o.ld_s16 + kc * 8 + half * 4);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(o.codes + row * o.ld_codes + kc * 128 + half * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) s.c[i] = p[i];
    s.s16 = 0u;
  }
  s.S = o.s128[row * o.ld_s128 + kc];
}

// Decode 64 elements to f16 and store them at dst (64 halves, 16-byte aligned).
__device__ __forceinline__ void decode_slice(int fmt, const Slice& s, _Float16* dst) {
  uint4* out = reinterpret_cast<uint4*>(dst);
  if (fmt == TJ2_NVFP4) {
    // inner scales as f16 pairs {s0, s1}, {s2, s3}
    half2_t sc01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s.s16, 1.0f, false);
    half2_t sc23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s.s16, 1.0f, true);
    const uint32_t w[8] = {s.c[0].x, s.c[0].y, s.c[0].z, s.c[0].w, s.c[1].x, s.c[1].y, s.c[1].z, s.c[1].w};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const half2_t sg = g == 0 ? half2_t{sc01[0], sc01[0]}
                       : g == 1 ? half2_t{sc01[1], sc01[1]}
                       : g == 2 ? half2_t{sc23[0], sc23[0]}
                                : half2_t{sc23[1], sc23[1]};
      uint32_t r[8];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t word = w[2 * g + d];
        half2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * sg;
        half2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * sg;
        half2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * sg;
        half2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * sg;
        r[4 * d + 0] = __builtin_bit_cast(uint32_t, q0);
        r[4 * d + 1] = __builtin_bit_cast(uint32_t, q1);
        r[4 * d + 2] = __builtin_bit_cast(uint32_t, q2);
        r[4 * d + 3] = __builtin_bit_cast(uint32_t, q3);
      }
      out[2 * g + 0] = make_uint4(r[0], r[1], r[2], r[3]);
      out[2 * g + 1] = make_uint4(r[4], r[5], r[6], r[7]);
    }
  } else {
    const uint32_t w[16] = {s.c[0].x, s.c[0].y, s.c[0].z, s.c[0].w, s.c[1].x, s.c[1].y, s.c[1].z, s.c[1].w,
                            s.c[2].x, s.c[2].y, s.c[2].z, s.c[2].w, s.c[3].x, s.c[3].y, s.c[3].z, s.c[3].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      half2_t a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * i], 1.0f, false);
      half2_t a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * i], 1.0f, true);
      half2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * i + 1], 1.0f, false);
      half2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * i + 1], 1.0f, true);
      out[i] = make_uint4(__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1),
                          __builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1));
    }
  }
}

__device__ __forceinline__ void chunk_of(const GemmKArgs& p, int c, int& seg, int& kc) {
  seg = (p.nseg > 1 && c >= p.seg[0].nchunks) ? 1 : 0;
  kc = seg ? c - p.seg[0].nchunks : c;
}

__global__ __launch_bounds__(256, 2) void gemm_nt_kernel(GemmKArgs p) {
  __shared__ __attribute__((aligned(16))) _Float16 lds_a[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) _Float16 lds_b[BN * LDS_STRIDE];
  __shared__ float sa[BM], sb[BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t rowA = m0 + lr, rowB = n0 + lr;
  const bool vA = rowA < p.I, vB = rowB < p.J;

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[i][j][t] = 0.0f;
  const float16_t zero = acc[0][0];

  Slice pa, pb;
  {
    int seg, kc;
    chunk_of(p, 0, seg, kc);
    load_slice(p.seg[seg].a, rowA, vA, kc, lh, pa);
    load_slice(p.seg[seg].b, rowB, vB, kc, lh, pb);
  }

  for (int c = 0; c < p.nchunks; ++c) {
    int seg, kc;
    chunk_of(p, c, seg, kc);
    const SegK& g = p.seg[seg];
    __syncthreads();  // previous chunk's LDS reads are done
    decode_slice(g.a.fmt, pa, lds_a + lr * LDS_STRIDE + lh * 64);
    decode_slice(g.b.fmt, pb, lds_b + lr * LDS_STRIDE + lh * 64);
    if (lh == 0) {
      sa[lr] = pa.S;
      sb[lr] = pb.S;
    }
    __syncthreads();
    if (c + 1 < p.nchunks) {
      int seg2, kc2;
      chunk_of(p, c + 1, seg2, kc2);
      load_slice(p.seg[seg2].a, rowA, vA, kc2, lh, pa);
      load_slice(p.seg[seg2].b, rowB, vB, kc2, lh, pb);
    }
    const int64_t krem = g.K - (int64_t)kc * BK;
    const int nk = (int)((krem < BK ? krem : BK) >> 4);

    float16_t part[2][2];
    const _Float16* a_base = lds_a + (wm * 64 + (lane & 31)) * LDS_STRIDE + (lane >> 5) * 8;
    const _Float16* b_base = lds_b + (wn * 64 + (lane & 31)) * LDS_STRIDE + (lane >> 5) * 8;
    {
      half8_t a0 = *reinterpret_cast<const half8_t*>(a_base);
      half8_t a1 = *reinterpret_cast<const half8_t*>(a_base + 32 * LDS_STRIDE);
      half8_t b0 = *reinterpret_cast<const half8_t*>(b_base);
      half8_t b1 = *reinterpret_cast<const half8_t*>(b_base + 32 * LDS_STRIDE);
      part[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, zero, 0, 0, 0);
      part[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, zero, 0, 0, 0);
      part[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, zero, 0, 0, 0);
      part[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, zero, 0, 0, 0);
    }
    for (int ks = 1; ks < nk; ++ks) {
      half8_t a0 = *reinterpret_cast<const half8_t*>(a_base + ks * 16);
      half8_t a1 = *reinterpret_cast<const half8_t*>(a_base + 32 * LDS_STRIDE + ks * 16);
      half8_t b0 = *reinterpret_cast<const half8_t*>(b_base + ks * 16);
      half8_t b1 = *reinterpret_cast<const half8_t*>(b_base + 32 * LDS_STRIDE + ks * 16);
      part[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, part[0][0], 0, 0, 0);
      part[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, part[0][1], 0, 0, 0);
      part[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, part[1][0], 0, 0, 0);
      part[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, part[1][1], 0, 0, 0);
    }
    // promote: acc += part * (S_A[row] * S_B[col])
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const float rb = sb[wn * 64 + tn * 32 + (lane & 31)];
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int r = wm * 64 + tm * 32 + 8 * (t >> 2) + 4 * (lane >> 5) + (t & 3);
          acc[tm][tn][t] = fmaf(part[tm][tn][t], sa[r] * rb, acc[tm][tn][t]);
        }
      }
    }
  }

  // epilogue
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    const int64_t col = n0 + wn * 64 + tn * 32 + (lane & 31);
    if (col >= p.J) continue;
    const int64_t ccol = p.col_map ? (int64_t)p.col_map[col] : col;
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int64_t row = m0 + wm * 64 + tm * 32 + 8 * (t >> 2) + 4 * (lane >> 5) + (t & 3);
        if (row >= p.I) continue;
        const float v = acc[tm][tn][t];
        if (p.c_bf16) {
          reinterpret_cast<uint16_t*>(p.C)[row * p.ldc + ccol] = (uint16_t)f32_to_bf16(v);
        } else {
          float* cp = reinterpret_cast<float*>(p.C) + row * p.ldc + ccol;
          *cp = p.accumulate ? *cp + v : v;
        }
      }
    }
  }
}

OperandK operand_of(const QView& v) {
  OperandK o;
  o.codes = v.codes;
  o.s16 = v.s16;
  o.s128 = v.s128;
  o.ld_codes = v.ld_codes;
  o.ld_s16 = v.ld_s16;
  o.ld_s128 = v.ld_s128;
  o.fmt = v.fmt;
  return o;
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  GemmKArgs k;
  k.nseg = p.nseg;
  k.nchunks = 0;
  for (int i = 0; i < 2; ++i) {
    if (i < p.nseg) {
      k.seg[i].a = operand_of(p.seg[i].a);
      k.seg[i].b = operand_of(p.seg[i].b);
      k.seg[i].K = p.seg[i].K;
      k.seg[i].nchunks = (int)((p.seg[i].K + BK - 1) / BK);
      k.nchunks += k.seg[i].nchunks;
    } else {
      k.seg[i] = k.seg[0];
      k.seg[i].nchunks = 0;
    }
  }
  k.I = p.I;
  k.J = p.J;
  k.C = p.C;
  k.ldc = p.ldc;
  k.col_map = p.col_map;
  k.c_bf16 = p.c_dtype == TJ2_BF16;
  k.accumulate = p.accumulate;
  dim3 grid((uint32_t)((p.J + BN - 1) / BN), (uint32_t)((p.I + BM - 1) / BM));
  hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(256), 0, s, k);
  return hipGetLastError();
}

}  // namespace tj2
