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
// 16-byte accesses).  Packed operands are prefetched two chunks ahead into
// registers; the eight 16-deep K steps of a chunk are unrolled with the LDS
// fragments of step k+1 read during step k; two workgroups per CU overlap one's
// decode with the other's MFMA.  Operand formats are template parameters (no
// runtime format branches); rows past the edge are clamped to the last row
// (their results are never stored), so loads never diverge.  Workgroups are
// numbered so that each of the 8 XCDs (own L2) gets a contiguous range of
// output tiles, N-fastest: consecutive tiles on one XCD share their A rows.
#include "tj2_device.h"
#include "tj2_internal.h"

namespace tj2 {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_STRIDE = BK + 8;  // f16 elements per LDS row
constexpr int F_NONE = -1;

struct OperandK {
  const uint8_t* codes;
  const uint8_t* s16;
  const float* s128;
  int64_t ld_codes, ld_s16, ld_s128;
};

struct SegK {
  OperandK a, b;
  int64_t K;
  int nchunks;
};

struct GemmKArgs {
  SegK seg[2];
  int nchunks;           // seg[0].nchunks + seg[1].nchunks
  int chunks_per_split;  // chunk range of split z: [z*cps, min((z+1)*cps, nchunks))
  int tiles_m, tiles_n, split;
  float* partial;        // split > 1: fp32 [split][I][J] partial sums
  int64_t I, J;
  void* C;
  int64_t ldc;
  const int32_t* col_map;
  int c_bf16;
  int accumulate;
};

// Packed slice of one thread: 64 consecutive K elements of one operand row.
template <int F>
struct Op;

template <>
struct Op<TJ2_NVFP4> {
  struct Slice {
    uint4 c0, c1;   // 64 E2M1 codes
    uint32_t s16;   // four E4M3 inner scales
    float S;        // outer scale of the chunk
  };
  static __device__ __forceinline__ void load(const OperandK& o, int64_t row, int kc, int half, Slice& s) {
    const uint8_t* cp = o.codes + row * o.ld_codes + kc * 64 + half * 32;
    s.c0 = *reinterpret_cast<const uint4*>(cp);
    s.c1 = *reinterpret_cast<const uint4*>(cp + 16);
    s.s16 = *reinterpret_cast<const uint32_t*>(o.s16 + row * o.ld_s16 + kc * 8 + half * 4);
    s.S = o.s128[row * o.ld_s128 + kc];
  }
  template <int BYTE>
  static __device__ __forceinline__ uint32_t q2(uint32_t word, half2_t sc) {
    half2_t q = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, BYTE) * sc;
    return __builtin_bit_cast(uint32_t, q);
  }
  // 64 f16 values q * s (exact) to dst (16-byte aligned)
  static __device__ __forceinline__ void decode(const Slice& s, _Float16* dst) {
    uint4* out = reinterpret_cast<uint4*>(dst);
    const half2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s.s16, 1.0f, false);
    const half2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s.s16, 1.0f, true);
    const half2_t sg[4] = {half2_t{s01[0], s01[0]}, half2_t{s01[1], s01[1]}, half2_t{s23[0], s23[0]},
                           half2_t{s23[1], s23[1]}};
    const uint32_t w[8] = {s.c0.x, s.c0.y, s.c0.z, s.c0.w, s.c1.x, s.c1.y, s.c1.z, s.c1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const half2_t sc = sg[i >> 1];
      out[i] = make_uint4(q2<0>(w[i], sc), q2<1>(w[i], sc), q2<2>(w[i], sc), q2<3>(w[i], sc));
    }
  }
};

template <>
struct Op<TJ2_FP8> {
  struct Slice {
    uint4 c[4];     // 64 E4M3 codes
    float S;
  };
  static __device__ __forceinline__ void load(const OperandK& o, int64_t row, int kc, int half, Slice& s) {
    const uint4* p = reinterpret_cast<const uint4*>(o.codes + row * o.ld_codes + kc * 128 + half * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) s.c[i] = p[i];
    s.S = o.s128[row * o.ld_s128 + kc];
  }
  template <bool HI>
  static __device__ __forceinline__ uint32_t e2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
  static __device__ __forceinline__ void decode(const Slice& s, _Float16* dst) {
    uint4* out = reinterpret_cast<uint4*>(dst);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = make_uint4(e2<false>(s.c[i].x), e2<true>(s.c[i].x), e2<false>(s.c[i].y), e2<true>(s.c[i].y));
      out[2 * i + 1] = make_uint4(e2<false>(s.c[i].z), e2<true>(s.c[i].z), e2<false>(s.c[i].w), e2<true>(s.c[i].w));
    }
  }
};

struct TileCtx {
  int64_t rowA, rowB;   // clamped source rows of this thread's loads
  int lr, lh, lane, wm, wn;
  _Float16* lds_a;
  _Float16* lds_b;
  float* sa;
  float* sb;
};

__device__ __forceinline__ half8_t ld8(const _Float16* p) { return *reinterpret_cast<const half8_t*>(p); }

// MFMA over one decoded chunk (nk 16-deep steps) and promotion into acc.
__device__ __forceinline__ void chunk_mfma(const TileCtx& t, int nk, float16_t (&acc)[2][2]) {
  const _Float16* ab = t.lds_a + (t.wm * 64 + (t.lane & 31)) * LDS_STRIDE + (t.lane >> 5) * 8;
  const _Float16* bb = t.lds_b + (t.wn * 64 + (t.lane & 31)) * LDS_STRIDE + (t.lane >> 5) * 8;
  float16_t part[2][2];
  if (nk == BK / 16) {
    half8_t fa[2][2], fb[2][2];
    fa[0][0] = ld8(ab);
    fa[0][1] = ld8(ab + 32 * LDS_STRIDE);
    fb[0][0] = ld8(bb);
    fb[0][1] = ld8(bb + 32 * LDS_STRIDE);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cb = ks & 1, nb = cb ^ 1;
      if (ks + 1 < BK / 16) {
        fa[nb][0] = ld8(ab + (ks + 1) * 16);
        fa[nb][1] = ld8(ab + 32 * LDS_STRIDE + (ks + 1) * 16);
        fb[nb][0] = ld8(bb + (ks + 1) * 16);
        fb[nb][1] = ld8(bb + 32 * LDS_STRIDE + (ks + 1) * 16);
      }
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
          part[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[cb][tm], fb[cb][tn],
                                                                ks == 0 ? float16_t{} : part[tm][tn], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
        part[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ld8(ab + tm * 32 * LDS_STRIDE),
                                                              ld8(bb + tn * 32 * LDS_STRIDE), float16_t{}, 0, 0, 0);
    for (int ks = 1; ks < nk; ++ks) {
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
          part[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ld8(ab + tm * 32 * LDS_STRIDE + ks * 16),
                                                                ld8(bb + tn * 32 * LDS_STRIDE + ks * 16),
                                                                part[tm][tn], 0, 0, 0);
    }
  }
  // promotion: acc += part * (S_A[row] * S_B[col]); rows t&3 of a lane are consecutive
  float rb[2];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) rb[tn] = t.sb[t.wn * 64 + tn * 32 + (t.lane & 31)];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 ra = *reinterpret_cast<const float4*>(t.sa + t.wm * 64 + tm * 32 + 8 * g + 4 * (t.lane >> 5));
      const float r4[4] = {ra.x, ra.y, ra.z, ra.w};
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[tm][tn][4 * g + q] = fmaf(part[tm][tn][4 * g + q], r4[q] * rb[tn], acc[tm][tn][4 * g + q]);
    }
  }
}

template <int FA, int FB>
__device__ __forceinline__ void stage_chunk(const TileCtx& t, const typename Op<FA>::Slice& a,
                                            const typename Op<FB>::Slice& b) {
  __syncthreads();  // the previous chunk's LDS reads are done
  Op<FA>::decode(a, t.lds_a + t.lr * LDS_STRIDE + t.lh * 64);
  Op<FB>::decode(b, t.lds_b + t.lr * LDS_STRIDE + t.lh * 64);
  if (t.lh == 0) {
    t.sa[t.lr] = a.S;
    t.sb[t.lr] = b.S;
  }
  __syncthreads();
}

// Chunks [kc0, kc1) of one segment, with a two-deep register prefetch.
template <int FA, int FB>
__device__ __forceinline__ void run_segment(const TileCtx& t, const SegK& g, int kc0, int kc1,
                                            float16_t (&acc)[2][2]) {
  if (kc0 >= kc1) return;
  typename Op<FA>::Slice a0, a1;
  typename Op<FB>::Slice b0, b1;
  Op<FA>::load(g.a, t.rowA, kc0, t.lh, a0);
  Op<FB>::load(g.b, t.rowB, kc0, t.lh, b0);
  if (kc0 + 1 < kc1) {
    Op<FA>::load(g.a, t.rowA, kc0 + 1, t.lh, a1);
    Op<FB>::load(g.b, t.rowB, kc0 + 1, t.lh, b1);
  }
  for (int kc = kc0; kc < kc1; kc += 2) {
    stage_chunk<FA, FB>(t, a0, b0);
    if (kc + 2 < kc1) {
      Op<FA>::load(g.a, t.rowA, kc + 2, t.lh, a0);
      Op<FB>::load(g.b, t.rowB, kc + 2, t.lh, b0);
    }
    int64_t krem = g.K - (int64_t)kc * BK;
    chunk_mfma(t, (int)((krem < BK ? krem : BK) >> 4), acc);
    if (kc + 1 >= kc1) break;
    stage_chunk<FA, FB>(t, a1, b1);
    if (kc + 3 < kc1) {
      Op<FA>::load(g.a, t.rowA, kc + 3, t.lh, a1);
      Op<FB>::load(g.b, t.rowB, kc + 3, t.lh, b1);
    }
    krem = g.K - (int64_t)(kc + 1) * BK;
    chunk_mfma(t, (int)((krem < BK ? krem : BK) >> 4), acc);
  }
}

template <int FA0, int FB0, int FA1, int FB1>
__global__ __launch_bounds__(256, 2) void gemm_nt_kernel(GemmKArgs p) {
  __shared__ __attribute__((aligned(16))) _Float16 lds_a[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) _Float16 lds_b[BN * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) float sa[BM];
  __shared__ __attribute__((aligned(16))) float sb[BN];

  // XCD-aware numbering: workgroup id w runs on XCD w % 8; give each XCD a
  // contiguous range of (tile, split) indices, tiles N-fastest.
  const uint32_t nwg = gridDim.x;
  uint32_t id = blockIdx.x;
  const uint32_t per_xcd = nwg / 8;
  if (id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;
  const uint32_t tiles = (uint32_t)(p.tiles_m * p.tiles_n);
  const uint32_t tile = id % tiles, z = id / tiles;
  const int64_t m0 = (int64_t)(tile / p.tiles_n) * BM, n0 = (int64_t)(tile % p.tiles_n) * BN;

  TileCtx t;
  const int tid = threadIdx.x;
  t.lane = tid & 63;
  const int wave = tid >> 6;
  t.wm = wave >> 1;
  t.wn = wave & 1;
  t.lr = tid >> 1;
  t.lh = tid & 1;
  t.rowA = min(m0 + t.lr, p.I - 1);
  t.rowB = min(n0 + t.lr, p.J - 1);
  t.lds_a = lds_a;
  t.lds_b = lds_b;
  t.sa = sa;
  t.sb = sb;

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = float16_t{};

  const int c_begin = (int)z * p.chunks_per_split;
  const int c_end = min(c_begin + p.chunks_per_split, p.nchunks);
  const int n0c = p.seg[0].nchunks;
  run_segment<FA0, FB0>(t, p.seg[0], c_begin, min(c_end, n0c), acc);
  if constexpr (FA1 != F_NONE) run_segment<FA1, FB1>(t, p.seg[1], max(c_begin, n0c) - n0c, c_end - n0c, acc);

  const int lane = t.lane;
  if (p.partial) {
    float* part_out = p.partial + (int64_t)z * p.I * p.J;
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const int64_t col = n0 + t.wn * 64 + tn * 32 + (lane & 31);
      if (col >= p.J) continue;
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t row = m0 + t.wm * 64 + tm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (row < p.I) part_out[row * p.J + col] = acc[tm][tn][e];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    const int64_t col = n0 + t.wn * 64 + tn * 32 + (lane & 31);
    if (col >= p.J) continue;
    const int64_t ccol = p.col_map ? (int64_t)p.col_map[col] : col;
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + t.wm * 64 + tm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row >= p.I) continue;
        const float v = acc[tm][tn][e];
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

// C[i, map(j)] (+)= sum_z partial[z][i][j]; one thread per 4 consecutive j.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int split, int64_t I,
                                                            int64_t J, void* C, int64_t ldc,
                                                            const int32_t* __restrict__ col_map, int c_bf16,
                                                            int accumulate) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t jq = (J + 3) / 4;
  const int64_t i = q / jq;
  if (i >= I) return;
  const int64_t j0 = (q - i * jq) * 4;
  float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t stride = I * J;
  const float* p = partial + i * J + j0;
  if (j0 + 4 <= J && (J & 3) == 0) {
    for (int z = 0; z < split; ++z) {
      float4 v = *reinterpret_cast<const float4*>(p + z * stride);
      s[0] += v.x; s[1] += v.y; s[2] += v.z; s[3] += v.w;
    }
  } else {
    for (int z = 0; z < split; ++z)
      for (int t = 0; t < 4; ++t)
        if (j0 + t < J) s[t] += p[z * stride + t];
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t j = j0 + t;
    if (j >= J) break;
    const int64_t cj = col_map ? (int64_t)col_map[j] : j;
    if (c_bf16) {
      reinterpret_cast<uint16_t*>(C)[i * ldc + cj] = (uint16_t)f32_to_bf16(s[t]);
    } else {
      float* cp = reinterpret_cast<float*>(C) + i * ldc + cj;
      *cp = accumulate ? *cp + s[t] : s[t];
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
  return o;
}

typedef void (*GemmKernel)(GemmKArgs);

GemmKernel pick_kernel(const GemmParams& p) {
  const int fa = p.seg[0].a.fmt, fb = p.seg[0].b.fmt;
  if (p.nseg == 2) {
    if (fa == TJ2_NVFP4 && fb == TJ2_NVFP4 && p.seg[1].a.fmt == TJ2_FP8 && p.seg[1].b.fmt == TJ2_FP8)
      return gemm_nt_kernel<TJ2_NVFP4, TJ2_NVFP4, TJ2_FP8, TJ2_FP8>;
    if (fa == TJ2_NVFP4 && fb == TJ2_NVFP4 && p.seg[1].a.fmt == TJ2_NVFP4 && p.seg[1].b.fmt == TJ2_NVFP4)
      return gemm_nt_kernel<TJ2_NVFP4, TJ2_NVFP4, TJ2_NVFP4, TJ2_NVFP4>;
    return nullptr;
  }
  if (fa == TJ2_NVFP4 && fb == TJ2_NVFP4) return gemm_nt_kernel<TJ2_NVFP4, TJ2_NVFP4, F_NONE, F_NONE>;
  if (fa == TJ2_NVFP4 && fb == TJ2_FP8) return gemm_nt_kernel<TJ2_NVFP4, TJ2_FP8, F_NONE, F_NONE>;
  if (fa == TJ2_FP8 && fb == TJ2_NVFP4) return gemm_nt_kernel<TJ2_FP8, TJ2_NVFP4, F_NONE, F_NONE>;
  if (fa == TJ2_FP8 && fb == TJ2_FP8) return gemm_nt_kernel<TJ2_FP8, TJ2_FP8, F_NONE, F_NONE>;
  return nullptr;
}

}  // namespace

int gemm_split(int64_t I, int64_t J, int64_t nchunks) {
  const int64_t tiles = ((I + BM - 1) / BM) * ((J + BN - 1) / BN);
  const int64_t target = 1024;  // workgroups: about two rounds of two per CU
  if (tiles >= target / 2 || nchunks < 8) return 1;
  int64_t split = (target + tiles - 1) / tiles;
  const int64_t max_by_depth = nchunks / 4;  // keep >= 4 chunks per split
  if (split > max_by_depth) split = max_by_depth;
  if (split > 64) split = 64;
  return split < 2 ? 1 : (int)split;
}

size_t gemm_workspace_bytes(int64_t I, int64_t J, int64_t nchunks) {
  const int split = gemm_split(I, J, nchunks);
  return split > 1 ? (size_t)split * (size_t)I * (size_t)J * sizeof(float) : 0;
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  GemmKernel kern = pick_kernel(p);
  if (!kern) return hipErrorInvalidValue;
  GemmKArgs k;
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
  int split = gemm_split(p.I, p.J, k.nchunks);
  if (split > 1 && (!p.partial || p.partial_bytes < (size_t)split * p.I * p.J * sizeof(float))) split = 1;
  k.chunks_per_split = (k.nchunks + split - 1) / split;
  split = (k.nchunks + k.chunks_per_split - 1) / k.chunks_per_split;  // no empty splits
  k.partial = split > 1 ? p.partial : nullptr;
  k.tiles_m = (int)((p.I + BM - 1) / BM);
  k.tiles_n = (int)((p.J + BN - 1) / BN);
  k.split = split;
  const uint32_t nwg = (uint32_t)k.tiles_m * (uint32_t)k.tiles_n * (uint32_t)split;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(256), 0, s, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 1) return e;
  const int64_t threads = p.I * ((p.J + 3) / 4);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, s, p.partial, split,
                     p.I, p.J, p.C, p.ldc, p.col_map, p.c_dtype == TJ2_BF16 ? 1 : 0, p.accumulate);
  return hipGetLastError();
}

}  // namespace tj2
