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
// into the accumulator with one multiply-add by S_A * S_B.  The products
// S_A * S_B of a chunk come from the fp32 outer-product MFMA
// (v_mfma_f32_32x32x1_2b_f32: two 32x32 blocks of a[i] * b[j] in fp32)
// straight in the accumulator layout, which leaves one VALU instruction per
// element and chunk.  CDNA4's
// block-scaled MFMA takes E8M0 scales per 32 elements, which cannot express an
// E4M3 scale per 16, hence the f16 decode.
//
// Kernel: a 256x128 output tile per 512-thread workgroup (one per CU); wave w
// owns rows 32w..32w+31 and all 128 columns (four 32x32 blocks of
// v_mfma_f32_32x32x16_f16).  A goes global -> registers -> MFMA: each wave
// decodes its own 32 rows (v_cvt_scalef32_pk_f16_fp4 / _fp8 at scale 1.0,
// exact, then v_pk_mul_f16 by the inner scale).  B (128 rows) is decoded once
// per workgroup into a double-buffered f16 LDS stage (rows padded to 272
// bytes: conflict-free 16-byte fragment reads) and read by all eight waves.
// Packed slices are prefetched one (A) and two to three (B) chunks ahead; a
// chunk is 32 MFMA issue slots per wave in a fixed order that spreads the
// decode, the promotion and the B staging over the slots, with one workgroup
// barrier per chunk.  Operand formats are template parameters (no runtime
// format branches); rows past the edge are clamped to the last row (their
// results are never stored), so loads never diverge.  Workgroups are numbered
// so that each of the 8 XCDs (own L2) gets a contiguous range of output tiles,
// N-fastest: consecutive tiles on one XCD share their A rows.  Results leave
// through LDS as 16-byte row pieces where the tile's columns are contiguous
// and aligned in the output (element stores otherwise).
//
// Image products (products of 2048 rows or more, when the caller gives room):
// B is decoded once into f16 chunk images laid out as the LDS stage, by the
// quantization that produces B or by a decode pass, and gemm_img_kernel (one
// K segment) and gemm_img2_kernel (the forward's NVFP4 + FP8 segments) copy
// each chunk's image into LDS with global_load_lds instead of decoding B.
#include "tj2_device.h"
#include "tj2_internal.h"

namespace tj2 {

namespace {

constexpr int BM = 256, BN = 128, BK = 128;
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
  // outlier-column products: J output columns in original order; column
  // outl[i] (sorted) takes B row i of b8 (FP8), the other columns in order take
  // the rows of seg[0].b (NVFP4); rest lists those other columns
  OperandK b8;
  const int32_t* outl;
  const int32_t* rest;
  int n_outl;
  // image products: B decoded once into f16 chunk images laid out as the LDS
  // stage ([tiles_n][nchunks] images of kImgChunkBytes) and its outer scales
  // S_B as [nchunks][bsc_ld] floats (bsc_ld = tiles_n * 128)
  const uint8_t* bimg;
  const float* bsc;
  int64_t bsc_ld;
};

// Packed slice of one thread, in a layout shared by both formats:
//  * A operand: 64 consecutive K elements (half of a 128-chunk) of one row.
//    NVFP4 uses q[0..1] (codes) and q[2].x (four inner scales); FP8 q[0..3].
//  * B operand: 32 consecutive K elements (a quarter chunk) of one row.
//    NVFP4 uses q[0] (codes), q[1].x (the aligned word holding its two inner
//    scales) and q[1].y (their bit offset in it); FP8 q[0..1].
struct Slice {
  uint4 q[4];
  float S;      // outer scale of the chunk
  uint32_t sc;  // NVFP6 A slice: its four inner scales
};

template <int F>
struct Op;

template <>
struct Op<TJ2_NVFP4> {
  static constexpr int kHalfLoads = 4;  // vector-memory instructions of load_half
  // rn = row * (outer blocks per row), below 2^32 for any operand that fits in memory (rows x
  // len / 128): codes at rn * 64 bytes (64-bit offsets: an operand's codes may exceed 4 GB),
  // inner scales at rn * 8, outer at rn
  static __device__ __forceinline__ void load_half(const OperandK& o, uint32_t rn, int kc, int half, Slice& s) {
    const uint8_t* cp = o.codes + (size_t)kc * 64 + ((size_t)rn * 64 + half * 32);
    s.q[0] = *reinterpret_cast<const uint4*>(cp);
    s.q[1] = *reinterpret_cast<const uint4*>(cp + 16);
    s.q[2].x = *reinterpret_cast<const uint32_t*>(o.s16 + (size_t)kc * 8 + ((size_t)rn * 8 + half * 4));
    s.S = (o.s128 + kc)[rn];
  }
  static __device__ __forceinline__ void load_quarter(const OperandK& o, uint32_t rn, int kc, int qt, Slice& s) {
    s.q[0] = *reinterpret_cast<const uint4*>(o.codes + (size_t)kc * 64 + ((size_t)rn * 64 + qt * 16));
    // the aligned word holding this quarter's two inner scales, and its shift: a
    // full-word load lands in the slice's own register (no extension on use)
    s.q[1].x = *reinterpret_cast<const uint32_t*>(o.s16 + (size_t)kc * 8 + ((size_t)rn * 8 + (qt >> 1) * 4));
    s.q[1].y = (uint32_t)(qt & 1) * 16u;
    s.S = (o.s128 + kc)[rn];
  }
  template <int BYTE>
  static __device__ __forceinline__ uint32_t q2(uint32_t word, half2_t sc) {
    half2_t q = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, BYTE) * sc;
    return __builtin_bit_cast(uint32_t, q);
  }
  // 8 codes (one word) times their inner scale: 8 exact f16 values
  static __device__ __forceinline__ half8_t dec8(uint32_t w, half2_t sc) {
    return __builtin_bit_cast(half8_t, make_uint4(q2<0>(w, sc), q2<1>(w, sc), q2<2>(w, sc), q2<3>(w, sc)));
  }
  static __device__ __forceinline__ void scales(uint32_t s16, half2_t (&sg)[4]) {
    const half2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s16, 1.0f, false);
    const half2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s16, 1.0f, true);
    sg[0] = half2_t{s01[0], s01[0]};
    sg[1] = half2_t{s01[1], s01[1]};
    sg[2] = half2_t{s23[0], s23[0]};
    sg[3] = half2_t{s23[1], s23[1]};
  }
  // piecewise decode used by the pipelined kernel: scale preparation, then one
  // 8-element fragment (A half slice) or unit (B quarter slice) at a time
  static __device__ __forceinline__ void prep_a(const Slice& s, half2_t (&sg)[4]) { scales(s.q[2].x, sg); }
  static __device__ __forceinline__ void prep_b(const Slice& s, half2_t (&sg)[4]) { scales(s.q[1].x >> s.q[1].y, sg); }
  template <int F>
  static __device__ __forceinline__ half8_t frag_a(const Slice& s, const half2_t (&sg)[4]) {
    const uint4& v = s.q[F >> 2];
    const uint32_t w = (F & 3) == 0 ? v.x : (F & 3) == 1 ? v.y : (F & 3) == 2 ? v.z : v.w;
    return dec8(w, sg[F >> 1]);
  }
  template <int U>
  static __device__ __forceinline__ half8_t unit_b(const Slice& s, const half2_t (&sg)[4]) {
    const uint4& v = s.q[0];
    const uint32_t w = U == 0 ? v.x : U == 1 ? v.y : U == 2 ? v.z : v.w;
    return dec8(w, sg[U >> 1]);
  }
  // half slice -> fragments f[i] = elements 8i..8i+7
  static __device__ __forceinline__ void decode_half(const Slice& s, half8_t (&f)[8]) {
    half2_t sg[4];
    scales(s.q[2].x, sg);
    const uint32_t w[8] = {s.q[0].x, s.q[0].y, s.q[0].z, s.q[0].w, s.q[1].x, s.q[1].y, s.q[1].z, s.q[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = dec8(w[i], sg[i >> 1]);
  }
  // quarter slice -> 32 f16 values at dst (16-byte aligned)
  static __device__ __forceinline__ void decode_quarter(const Slice& s, _Float16* dst) {
    half2_t sg[4];
    scales(s.q[1].x >> s.q[1].y, sg);
    half8_t* out = reinterpret_cast<half8_t*>(dst);
    out[0] = dec8(s.q[0].x, sg[0]);
    out[1] = dec8(s.q[0].y, sg[0]);
    out[2] = dec8(s.q[0].z, sg[1]);
    out[3] = dec8(s.q[0].w, sg[1]);
  }
};

template <>
struct Op<TJ2_FP8> {
  static constexpr int kHalfLoads = 5;
  // rn = row * (outer blocks per row): codes at rn * 128 bytes, outer scales at rn
  static __device__ __forceinline__ void load_half(const OperandK& o, uint32_t rn, int kc, int half, Slice& s) {
    const uint4* p = reinterpret_cast<const uint4*>(o.codes + (size_t)kc * 128 + ((size_t)rn * 128 + half * 64));
#pragma unroll
    for (int i = 0; i < 4; ++i) s.q[i] = p[i];
    s.S = (o.s128 + kc)[rn];
  }
  static __device__ __forceinline__ void load_quarter(const OperandK& o, uint32_t rn, int kc, int qt, Slice& s) {
    const uint4* p = reinterpret_cast<const uint4*>(o.codes + (size_t)kc * 128 + ((size_t)rn * 128 + qt * 32));
    s.q[0] = p[0];
    s.q[1] = p[1];
    s.S = (o.s128 + kc)[rn];
  }
  template <bool HI>
  static __device__ __forceinline__ uint32_t e2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
  static __device__ __forceinline__ half8_t dec8(uint32_t w0, uint32_t w1) {
    return __builtin_bit_cast(half8_t, make_uint4(e2<false>(w0), e2<true>(w0), e2<false>(w1), e2<true>(w1)));
  }
  static __device__ __forceinline__ void prep_a(const Slice&, half2_t (&)[4]) {}
  static __device__ __forceinline__ void prep_b(const Slice&, half2_t (&)[4]) {}
  template <int F>
  static __device__ __forceinline__ half8_t frag_a(const Slice& s, const half2_t (&)[4]) {
    const uint4& v = s.q[F >> 1];
    return (F & 1) ? dec8(v.z, v.w) : dec8(v.x, v.y);
  }
  template <int U>
  static __device__ __forceinline__ half8_t unit_b(const Slice& s, const half2_t (&)[4]) {
    const uint4& v = s.q[U >> 1];
    return (U & 1) ? dec8(v.z, v.w) : dec8(v.x, v.y);
  }
  static __device__ __forceinline__ void decode_half(const Slice& s, half8_t (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = dec8(s.q[i].x, s.q[i].y);
      f[2 * i + 1] = dec8(s.q[i].z, s.q[i].w);
    }
  }
  static __device__ __forceinline__ void decode_quarter(const Slice& s, _Float16* dst) {
    half8_t* out = reinterpret_cast<half8_t*>(dst);
    out[0] = dec8(s.q[0].x, s.q[0].y);
    out[1] = dec8(s.q[0].z, s.q[0].w);
    out[2] = dec8(s.q[1].x, s.q[1].y);
    out[3] = dec8(s.q[1].z, s.q[1].w);
  }
};

// NVFP6 A operand of the FP6 x FP4 products: E2M3 elements stored as E4M3FN
// bytes (rn * 128 bytes per row block, like FP8) under E4M3 inner scales per 16
// (rn * 8, like NVFP4).  The fp8 -> f16 conversion is exact on them, and an
// E2M3 value (4 significant bits) times an E4M3 scale (4) is exact in f16.
template <>
struct Op<TJ2_NVFP6> {
  static constexpr int kHalfLoads = 6;
  static __device__ __forceinline__ void load_half(const OperandK& o, uint32_t rn, int kc, int half, Slice& s) {
    const uint4* p = reinterpret_cast<const uint4*>(o.codes + (size_t)kc * 128 + ((size_t)rn * 128 + half * 64));
#pragma unroll
    for (int i = 0; i < 4; ++i) s.q[i] = p[i];
    s.sc = *reinterpret_cast<const uint32_t*>(o.s16 + (size_t)kc * 8 + ((size_t)rn * 8 + half * 4));
    s.S = (o.s128 + kc)[rn];
  }
  static __device__ __forceinline__ void prep_a(const Slice& s, half2_t (&sg)[4]) { Op<TJ2_NVFP4>::scales(s.sc, sg); }
  template <int F>
  static __device__ __forceinline__ half8_t frag_a(const Slice& s, const half2_t (&sg)[4]) {
    const uint4& v = s.q[F >> 1];
    const half8_t e = (F & 1) ? Op<TJ2_FP8>::dec8(v.z, v.w) : Op<TJ2_FP8>::dec8(v.x, v.y);
    const _Float16 c = sg[F >> 1][0];
    return e * half8_t{c, c, c, c, c, c, c, c};
  }
};

__device__ __forceinline__ half8_t ld8(const _Float16* p) { return *reinterpret_cast<const half8_t*>(p); }

// B fragments are read D MFMA slots before use, in a ring of frag_ring(D)
// registers (32 % ring == 0 so ring positions carry over between chunks).
// D = 5 (3 to 7 measure the same).
constexpr int frag_ring(int d) { return d < 4 ? 4 : 8; }
constexpr int kFragAheadSlots = 5;

typedef float float16v_t __attribute__((ext_vector_type(16)));
typedef float float32v_t __attribute__((ext_vector_type(32)));

// Shared memory: two decoded f16 stages of the B tile and four-deep rings of
// the outer scales of both operands (a chunk's scales are read one chunk later).
struct Smem {
  _Float16 b[2][BN * LDS_STRIDE];
  float sa[4][BM];
  float sb[4][BN];
};

// Output staging after the K loop, in the same memory: each wave's 32x128 fp32
// results (rows padded to 136 words: the two lane halves, four rows apart,
// write disjoint bank halves).
constexpr int OUT_STRIDE = BN + 8;
union SmemAll {
  Smem loop;
  float out[BM / 32][32][OUT_STRIDE];
};

// Per-thread roles.  Wave w owns output rows 32w..32w+31 of the 256x128 tile
// and all 128 columns (four 32x32 blocks).  A rows go global -> registers ->
// MFMA: lane l loads row 32w + (l & 31), K half h = l >> 5 of each chunk, and
// MFMA step ks consumes K elements 64h + 8ks .. 64h + 8ks + 7 (the same
// permutation of K is applied to B, so the sum is unchanged).  B rows are
// decoded once per workgroup into LDS: thread t stages row t >> 2, quarter t & 3.
struct Ctx {
  uint32_t arn[2], brn[2];  // clamped source row * outer blocks per row, per segment
  bool b8;                  // outlier-column products: this thread stages an FP8 row (from p.b8)
  int ah, bq;               // A half, B quarter
  int lane, w;
  int n0c;                  // chunks of segment 0
  int c_begin;              // first chunk of this workgroup
};

template <int FA0, int FB0, int FA1, int FB1>
struct Fmt {
  // the A slice / B slice of workgroup-local chunk `it` (if it exists)
  // (an index past the range reloads the last chunk: branch-free, the data is unused)
  static __device__ __forceinline__ void fetch_a(const GemmKArgs& p, const Ctx& t, int it, int n, Slice& a) {
    const int g = t.c_begin + min(it, n - 1);
    if (FA1 == F_NONE || g < t.n0c) Op<FA0>::load_half(p.seg[0].a, t.arn[0], g, t.ah, a);
    else if constexpr (FA1 != F_NONE) Op<FA1>::load_half(p.seg[1].a, t.arn[1], g - t.n0c, t.ah, a);
  }
  static __device__ __forceinline__ void fetch_b(const GemmKArgs& p, const Ctx& t, int it, int n, Slice& b) {
    const int g = t.c_begin + min(it, n - 1);
    if (FA1 == F_NONE || g < t.n0c) Op<FB0>::load_quarter(p.seg[0].b, t.brn[0], g, t.bq, b);
    else if constexpr (FA1 != F_NONE) Op<FB1>::load_quarter(p.seg[1].b, t.brn[1], g - t.n0c, t.bq, b);
  }
};

// Outlier-column products: A NVFP4 (or NVFP6); B rows NVFP4 (seg[0].b) or FP8 (b8) per thread.
template <int FA>
struct FmtMixB {
  static __device__ __forceinline__ void fetch_a(const GemmKArgs& p, const Ctx& t, int it, int n, Slice& a) {
    Op<FA>::load_half(p.seg[0].a, t.arn[0], t.c_begin + min(it, n - 1), t.ah, a);
  }
  // Branch-free: every thread issues the same loads from addresses selected by its
  // format (an NVFP4 thread's second 16 bytes and an FP8 thread's inner scales
  // are read from valid addresses and ignored).
  static __device__ __forceinline__ void fetch_b(const GemmKArgs& p, const Ctx& t, int it, int n, Slice& b) {
    const int g = t.c_begin + min(it, n - 1);
    const uint8_t* c4 = p.seg[0].b.codes + (size_t)g * 64 + ((size_t)t.brn[0] * 64 + t.bq * 16);
    const uint8_t* c8 = p.b8.codes + (size_t)g * 128 + ((size_t)t.brn[1] * 128 + t.bq * 32);
    const uint8_t* c = t.b8 ? c8 : c4;
    b.q[0] = *reinterpret_cast<const uint4*>(c);
    b.q[1] = *reinterpret_cast<const uint4*>(t.b8 ? c8 + 16 : c4);
    b.q[2].x = *reinterpret_cast<const uint32_t*>(p.seg[0].b.s16 + (size_t)g * 8 + ((size_t)t.brn[0] * 8 + (t.bq >> 1) * 4));
    b.q[2].y = (uint32_t)(t.bq & 1) * 16u;
    b.S = t.b8 ? (p.b8.s128 + g)[t.brn[1]] : (p.seg[0].b.s128 + g)[t.brn[0]];
  }
};

// Outer scales of one 32x32 output block of a chunk, as this lane needs them:
// S_B of its column and S_A of its 16 rows (rows 8g + 4*(lane/32) + q hold
// element 4g + q).
struct Scl {
  float rb;
  float4 ra[4];
};

__device__ __forceinline__ void read_scl(const Smem& sm, const Ctx& t, int slot, int tn, Scl& c) {
  c.rb = sm.sb[slot][tn * 32 + (t.lane & 31)];
#pragma unroll
  for (int g = 0; g < 4; ++g)
    c.ra[g] = *reinterpret_cast<const float4*>(&sm.sa[slot][t.w * 32 + 8 * g + 4 * (t.lane >> 5)]);
}

template <int E>
__device__ __forceinline__ void promote_elem(const Scl& c, const float16v_t& part, float (&acc)[16]) {
  const float4& r = c.ra[E >> 2];
  const float ra = (E & 3) == 0 ? r.x : (E & 3) == 1 ? r.y : (E & 3) == 2 ? r.z : r.w;
  acc[E] = fmaf(part[E], ra * c.rb, acc[E]);
}

__device__ __forceinline__ void barrier_lds() {
  // LDS writes of this wave are complete; global prefetches may stay in flight
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Operand formats of the two K segments: the A slice of a chunk and the B
// quarter staged for the next chunk are in segment 1 when the flag says so.
template <int FA0, int FB0, int FA1, int FB1>
struct Fmts {
  static constexpr bool kMixedA = FA1 != F_NONE && FA1 != FA0;
  static constexpr bool kMixedB = FA1 != F_NONE && FB1 != FB0;
  static constexpr int kFA1 = FA1 == F_NONE ? FA0 : FA1;
  static constexpr int kFB1 = FA1 == F_NONE ? FB0 : FB1;
  static __device__ __forceinline__ void prep_a(const Slice& a, half2_t (&sg)[4]) { Op<FA0>::prep_a(a, sg); }
  static __device__ __forceinline__ void prep_b(const Slice& b, half2_t (&sg)[4]) { Op<FB0>::prep_b(b, sg); }
  template <int F>
  static __device__ __forceinline__ half8_t frag_a(const Slice& a, const half2_t (&sg)[4], bool seg1) {
    if constexpr (kMixedA) {
      if (seg1) return Op<kFA1>::template frag_a<F>(a, sg);
    }
    return Op<FA0>::template frag_a<F>(a, sg);
  }
  template <int U>
  static __device__ __forceinline__ half8_t unit_b(const Slice& b, const half2_t (&sg)[4], bool seg1) {
    if constexpr (kMixedB) {
      if (seg1) return Op<kFB1>::template unit_b<U>(b, sg);
    }
    return Op<FB0>::template unit_b<U>(b, sg);
  }
};

template <int FA>
struct FmtsMixB {
  static __device__ __forceinline__ void prep_a(const Slice& a, half2_t (&sg)[4]) { Op<FA>::prep_a(a, sg); }
  // the NVFP4 inner scales sit in q[2].x of a B slice here (q[1] holds FP8 codes)
  static __device__ __forceinline__ void prep_b(const Slice& b, half2_t (&sg)[4]) {
    Op<TJ2_NVFP4>::scales(b.q[2].x >> b.q[2].y, sg);
  }
  template <int F>
  static __device__ __forceinline__ half8_t frag_a(const Slice& a, const half2_t (&sg)[4], bool) {
    return Op<FA>::template frag_a<F>(a, sg);
  }
  // both decodes, selected per lane (no divergent branch)
  template <int U>
  static __device__ __forceinline__ half8_t unit_b(const Slice& b, const half2_t (&sg)[4], bool fp8) {
    const half8_t v8 = Op<TJ2_FP8>::template unit_b<U>(b, sg);
    const half8_t v4 = Op<TJ2_NVFP4>::template unit_b<U>(b, sg);
    return fp8 ? v8 : v4;
  }
};

// One chunk as 32 issue slots (block tn = q / 8, K step ks = q % 8).  Slot q:
// in block 0 decodes A fragment q + 1 of this chunk from the wave's A slice (the
// previous chunk's last MFMA reading that fragment has issued; fragment 0 was
// decoded in the previous chunk's last slot, from this chunk's slice), reads the B
// fragment of slot q + kFragAhead, issues one MFMA into the block's partial
// (blocks alternate between two partials), promotes two or three elements of
// the previous block at K-steps 2-7 (block 3 of the previous chunk during
// block 0; before the first chunk that partial and its scales are zero) with
// the scale products of blocks 0-1 and 2-3 issued at slots 8 and 24, and
// stages the next chunk's B quarter into the other LDS stage at slots 9, 15,
// 20, 25, away from block 0's A decode, and its B outer scales at slot 3
// (after the last chunk this writes unused data).  At slot 8 the A
// slice is refilled with the next chunk (fetch_a); its S_A was kept from the
// chunk start.  The workgroup barrier (sync) sits in
// slot 32 - kFragAhead, once the next stage is written and this chunk's last
// fragment read has been issued, so the last slots already read the next
// chunk's first fragments.  A scheduling barrier after each slot keeps this
// order.  Chunks past the end of a segment's K are zero in the padded operands,
// so every chunk runs all steps.
template <class FM, int kFragAhead, class FETCH_A, class SYNC>
__device__ __forceinline__ void chunk(Smem& sm, const Ctx& t, int it, bool aseg1, bool bseg1, half8_t (&af)[8],
                                      half2_t (&sga)[4], half8_t (&bf)[frag_ring(kFragAhead)], float (&acc)[4][16],
                                      float16v_t (&part)[2], float32v_t& smat, Slice& a, const Slice& nb,
                                      FETCH_A&& fetch_a, SYNC&& sync) {
  const _Float16* bb = sm.b[it & 1] + (t.lane & 31) * LDS_STRIDE + (t.lane >> 5) * 64;
  const _Float16* bn = sm.b[(it + 1) & 1] + (t.lane & 31) * LDS_STRIDE + (t.lane >> 5) * 64;
  _Float16* bdst = sm.b[(it + 1) & 1] + (threadIdx.x >> 2) * LDS_STRIDE + t.bq * 32;
  constexpr int kFragRing = frag_ring(kFragAhead);
  half2_t sgb[4];
  const float sa = a.S;  // S_A of this lane's row (both lane halves load the same row)
  float sbp = 0.0f;
  static_for<32>([&](auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    constexpr int tn = q / 8, ks = q % 8;
    // A fragment q + 1 is decoded in slot q, one slot before its first MFMA;
    // fragment 0 of the next chunk in slot 31 (after its last use in slot 24)
    if constexpr (q < 7) af[q + 1] = FM::template frag_a<q + 1>(a, sga, aseg1);
    if constexpr (q == 8) fetch_a(a);
    if constexpr (q == 30) FM::prep_a(a, sga);  // the next chunk's slice
    if constexpr (q == 31) af[0] = FM::template frag_a<0>(a, sga, aseg1);
    if constexpr (q == 32 - kFragAhead) sync();
    constexpr int qf = q + kFragAhead;  // fragment read in this slot
    if constexpr (qf < 32) bf[qf % kFragRing] = ld8(bb + (qf / 8) * 32 * LDS_STRIDE + (qf % 8) * 8);
    else bf[qf % kFragRing] = ld8(bn + (qf - 32) * 8);
    // S_B of the column pair's two blocks: lanes 0-31 block 2p, lanes 32-63 block 2p + 1
    if constexpr (q == 4 || q == 20) sbp = sm.sb[it & 3][(q == 4 ? 0 : 64) + t.lane];
    // outer-scale products S_A[row] * S_B[col] of blocks 0-1 (slot 8) and 2-3 (slot 24) in the
    // accumulator layout: the 2-block fp32 outer product (block b in elements 16b..16b+15)
    if constexpr (q == 8 || q == 24) smat = __builtin_amdgcn_mfma_f32_32x32x1f32(sa, sbp, float32v_t{}, 0, 0, 0);
    part[tn & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks], bf[q % kFragRing], ks == 0 ? float16v_t{} : part[tn & 1],
                                                          0, 0, 0);
    if constexpr (ks >= 2) {
      // elements [lo, hi) of the previous block at K-step ks (2..7): 3,3,3,3,2,2 (its last MFMA
      // has completed; block 3 of the previous chunk during block 0)
      constexpr int pb = tn > 0 ? tn - 1 : 3;
      constexpr int lo = ks <= 6 ? 3 * (ks - 2) : 14, hi = ks < 6 ? lo + 3 : lo + 2;
      static_for<hi - lo>([&](auto i) __attribute__((always_inline)) {
        constexpr int e = lo + decltype(i)::value;
        acc[pb][e] = fmaf(part[pb & 1][e], smat[16 * (pb & 1) + e], acc[pb][e]);
      });
    }
    if constexpr (q == 1) FM::prep_b(nb, sgb);
    if constexpr (q == 9 || q == 15 || q == 20 || q == 25) {
      constexpr int u = q == 9 ? 0 : q == 15 ? 1 : q == 20 ? 2 : 3;
      *reinterpret_cast<half8_t*>(bdst + u * 8) = FM::template unit_b<u>(nb, sgb, bseg1);
    }
    if constexpr (q == 3) sm.sb[(it + 1) & 3][threadIdx.x >> 2] = nb.S;
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Stage the B quarter of the first chunk of the range (format FB).
template <int FB>
__device__ __forceinline__ void stage_first_b(Smem& sm, const Ctx& t, const Slice& b) {
  Op<FB>::decode_quarter(b, sm.b[0] + (threadIdx.x >> 2) * LDS_STRIDE + t.bq * 32);
  sm.sb[0][threadIdx.x >> 2] = b.S;
}

// A chunk of the second K segment (the FP8 outlier channels, at most a few
// chunks per tile): loaded, decoded and multiplied without pipelining, each
// block promoted right after its eight K steps.
template <int FA, int FB>
__device__ __forceinline__ void tail_chunk(const GemmKArgs& p, Smem& sm, const Ctx& t, int g, float (&acc)[4][16]) {
  Slice a, b;
  Op<FA>::load_half(p.seg[1].a, t.arn[1], g, t.ah, a);
  Op<FB>::load_quarter(p.seg[1].b, t.brn[1], g, t.bq, b);
  barrier_lds();  // every wave is done with the previous chunk's stage and scales
  Op<FB>::decode_quarter(b, sm.b[0] + (threadIdx.x >> 2) * LDS_STRIDE + t.bq * 32);
  sm.sb[0][threadIdx.x >> 2] = b.S;
  sm.sa[0][t.w * 32 + (t.lane & 31)] = a.S;
  half8_t af[8];
  Op<FA>::decode_half(a, af);
  barrier_lds();
  const _Float16* bb = sm.b[0] + (t.lane & 31) * LDS_STRIDE + (t.lane >> 5) * 64;
  Scl scl;
  read_scl(sm, t, 0, 0, scl);
  // B fragments are read one block ahead of their MFMAs
  half8_t bfr[2][BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) bfr[0][ks] = ld8(bb + ks * 8);
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) {
    if (tn < 3) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) bfr[(tn + 1) & 1][ks] = ld8(bb + (tn + 1) * 32 * LDS_STRIDE + ks * 8);
    }
    float16v_t part = float16v_t{};
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
      part = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks], bfr[tn & 1][ks], part, 0, 0, 0);
    scl.rb = sm.sb[0][tn * 32 + (t.lane & 31)];
    static_for<16>([&](auto e) __attribute__((always_inline)) {
      promote_elem<decltype(e)::value>(scl, part, acc[tn]);
    });
  }
}

// Workgroup: 512 threads (8 waves), one 256x128 output tile, the chunk range of split z.
// first index i in [0, n) with a[i] >= v (a sorted ascending), n if none
__device__ __forceinline__ int lower_bound(const int32_t* a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to the nearest even bf16 (v_cvt_pk_bf16_f32; the
// kernels' float mode keeps denormals), a in the low half.  Equal to
// f32_to_bf16 on finite values.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Output of one 256x128 tile from the accumulators (MIXB: the outlier-column
// mapping of the staged rows: lo, c1, r0, ncols as set up by the kernel).
template <bool MIXB>
__device__ __forceinline__ void store_tile(const GemmKArgs& p, float (*out)[32][OUT_STRIDE], const Ctx& t, int64_t m0,
                                           int64_t n0, uint32_t z, const float (&acc)[4][16], int lo, int c1, int r0,
                                           int ncols) {
  // Output: lane holds rows 8g + 4*(lane/32) + q (element 4g + q) of the wave's
  // 32 rows, column tn*32 + (lane & 31) of block tn (staged LDS row; for
  // outlier-column products mapped back to the original column).
  const int lane = t.lane;
  const int64_t rw = m0 + t.w * 32 + 4 * (lane >> 5);
  const bool full_rows = m0 + BM <= p.I;
  int64_t ocol[4];
  bool ok[4];
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) {
    const int rho = tn * 32 + (lane & 31);
    if constexpr (MIXB) {
      ok[tn] = rho < ncols;
      ocol[tn] = !ok[tn] ? 0 : rho < c1 ? (int64_t)p.rest[r0 + rho] : (int64_t)p.outl[lo + rho - c1];
    } else {
      ocol[tn] = n0 + rho;
      ok[tn] = ocol[tn] < p.J;
    }
  }
  // Tiles whose 128 columns are contiguous and 16-byte aligned in the output go
  // through LDS and leave as 16-byte row pieces (8 bf16 or 4 fp32 per store)
  // instead of one 2- or 4-byte store per element.  An outlier-column tile's
  // columns are the full range [n0, n0 + 128) in another order (its non-outlier
  // columns and its outlier columns, both ascending), so its results are
  // placed in output order on the way into LDS.
  {
    const bool to_partial = p.partial != nullptr;
    const int64_t ld = to_partial ? p.J : p.ldc;
    const bool bf = !to_partial && p.c_bf16;
    const uintptr_t base_addr = to_partial ? (uintptr_t)p.partial : (uintptr_t)p.C;
    if (n0 + BN <= p.J && (MIXB || to_partial || !p.col_map) && (ld & (bf ? 7 : 3)) == 0 &&
        (base_addr & 15) == 0) {
      barrier_lds();  // every wave is done with the last chunk's B stage
      float(&st)[32][OUT_STRIDE] = out[t.w];
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        // output column within the tile (clamped: a plan that breaks its contract cannot
        // move a write outside the wave's staging rows)
        const int lc = MIXB ? min(max((int)(ocol[tn] - n0), 0), BN - 1) : tn * 32 + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) st[8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)][lc] = acc[tn][e];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's writes are visible to its lanes
      __builtin_amdgcn_wave_barrier();
      const int64_t row0 = m0 + t.w * 32;
      // rows of the wave's 32 inside the output (fewer in a last, partial row tile)
      const int rows_here = (int)min(p.I - row0, (int64_t)32);
      // Each lane forms its 64-bit output address once and steps it by a uniform
      // row stride per pass (a 64-bit row x stride product per pass costs three
      // quarter-rate multiplies), and bf16 pairs come from the hardware
      // conversion (one instruction per two values).
      if (bf) {
        // lane: 8 columns of one of four rows per pass
        const int rl = lane >> 4, c0 = (lane & 15) * 8;
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.C) + (row0 + rl) * ld + n0 + c0;
        const int64_t step = 4 * ld;
#pragma unroll
        for (int r = 0; r < 8; ++r, dst += step) {
          const int row = 4 * r + rl;
          const float4 u = *reinterpret_cast<const float4*>(&st[row][c0]);
          const float4 v = *reinterpret_cast<const float4*>(&st[row][c0 + 4]);
          uint4 o;
          o.x = pk_bf16(u.x, u.y);
          o.y = pk_bf16(u.z, u.w);
          o.z = pk_bf16(v.x, v.y);
          o.w = pk_bf16(v.z, v.w);
          if (row < rows_here) *reinterpret_cast<uint4*>(dst) = o;
        }
      } else {
        float* base = to_partial ? p.partial + (int64_t)z * p.I * p.J : reinterpret_cast<float*>(p.C);
        const bool add = !to_partial && p.accumulate;
        // lane: 4 columns of one of two rows per pass
        const int rl = lane >> 5, c0 = (lane & 31) * 4;
        float* dst0 = base + (row0 + rl) * ld + n0 + c0;
        const int64_t step = 2 * ld;
#pragma unroll
        for (int r = 0; r < 16; ++r, dst0 += step) {
          const int row = 2 * r + rl;
          float4 v = *reinterpret_cast<const float4*>(&st[row][c0]);
          if (row < rows_here) {
            float4* dst = reinterpret_cast<float4*>(dst0);
            if (add) {
              const float4 o = *dst;
              v.x = o.x + v.x;
              v.y = o.y + v.y;
              v.z = o.z + v.z;
              v.w = o.w + v.w;
            }
            *dst = v;
          }
        }
      }
      return;
    }
  }
  if (p.partial) {
    float* base = p.partial + (int64_t)z * p.I * p.J + rw * p.J;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      if (!ok[tn]) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int dr = 8 * (e >> 2) + (e & 3);
        if (full_rows || rw + dr < p.I) base[dr * p.J + ocol[tn]] = acc[tn][e];
      }
    }
    return;
  }
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) {
    if (!ok[tn]) continue;
    const int64_t ccol = (!MIXB && p.col_map) ? (int64_t)p.col_map[ocol[tn]] : ocol[tn];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int dr = 8 * (e >> 2) + (e & 3);
      if (!full_rows && rw + dr >= p.I) continue;
      const int64_t off = (rw + dr) * p.ldc + ccol;
      const float v = acc[tn][e];
      if (p.c_bf16) {
        reinterpret_cast<uint16_t*>(p.C)[off] = (uint16_t)f32_to_bf16(v);
      } else {
        float* cp = reinterpret_cast<float*>(p.C) + off;
        *cp = p.accumulate ? *cp + v : v;
      }
    }
  }
}

template <int FA0, int FB0, int FA1, int FB1, bool MIXB>
__global__ __launch_bounds__(512, 1) void gemm_nt_kernel(GemmKArgs p) {
  __shared__ __attribute__((aligned(16))) SmemAll smem;
  Smem& sm = smem.loop;

  // XCD-aware numbering: workgroup id w runs on XCD w % 8; give each XCD a
  // contiguous range of (tile, split) indices, tiles N-fastest.
  const uint32_t nwg = gridDim.x;
  uint32_t id = blockIdx.x;
  const uint32_t per_xcd = nwg / 8;
  if (id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;
  const uint32_t tiles = (uint32_t)(p.tiles_m * p.tiles_n);
  const uint32_t tile = id % tiles, z = id / tiles;
  const int64_t m0 = (int64_t)(tile / p.tiles_n) * BM, n0 = (int64_t)(tile % p.tiles_n) * BN;

  Ctx t;
  t.lane = threadIdx.x & 63;
  t.w = threadIdx.x >> 6;
  t.ah = t.lane >> 5;
  t.bq = threadIdx.x & 3;
  const uint32_t arow = (uint32_t)min(m0 + t.w * 32 + (t.lane & 31), p.I - 1);
  const uint32_t brow = (uint32_t)min(n0 + (int64_t)(threadIdx.x >> 2), p.J - 1);
#pragma unroll
  for (int sgi = 0; sgi < 2; ++sgi) {
    t.arn[sgi] = arow * (uint32_t)p.seg[sgi].a.ld_s128;
    t.brn[sgi] = brow * (uint32_t)p.seg[sgi].b.ld_s128;
  }
  t.b8 = false;
  // Outlier-column products: the tile's output columns [n0, n0 + ncols) are
  // staged as LDS rows [0, c1) = its non-outlier columns in order (B rows r0..),
  // then rows [c1, ncols) = its outlier columns (FP8 rows lo..), so at most one
  // wave mixes the two formats; the epilogue maps rows back to columns.
  int lo = 0, c1 = BN, r0 = 0, ncols = BN;
  if constexpr (MIXB) {
    lo = lower_bound(p.outl, p.n_outl, (int)n0);
    const int hi = lower_bound(p.outl, p.n_outl, (int)min(n0 + BN, p.J));
    ncols = (int)min((int64_t)BN, p.J - n0);
    c1 = ncols - (hi - lo);
    r0 = (int)n0 - lo;
    const int rho = threadIdx.x >> 2;
    t.b8 = rho >= c1 && rho < ncols;
    const int64_t n1 = p.J - p.n_outl;  // rows of the NVFP4 B operand
    t.brn[0] = (uint32_t)min((int64_t)(r0 + rho), n1 - 1) * (uint32_t)p.seg[0].b.ld_s128;
    t.brn[1] = (uint32_t)min(lo + max(rho - c1, 0), p.n_outl - 1) * (uint32_t)p.b8.ld_s128;
  }
  t.n0c = p.seg[0].nchunks;
  t.c_begin = (int)z * p.chunks_per_split;
  const int n = min(t.c_begin + p.chunks_per_split, p.nchunks) - t.c_begin;

  float acc[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;

  // chunks [0, s1) of the range are segment 0 (pipelined), [s1, n) segment 1
  const int s1 = FA1 == F_NONE ? n : min(max(t.n0c - t.c_begin, 0), n);
  if (s1 > 0) {
    using F = std::conditional_t<MIXB, FmtMixB<FA0>, Fmt<FA0, FB0, F_NONE, F_NONE>>;
    using FM = std::conditional_t<MIXB, FmtsMixB<FA0>, Fmts<FA0, FB0, F_NONE, F_NONE>>;
    Slice a, b1, b2;
    half8_t af[8];
    half2_t sga[4];
    float16v_t part[2];
    part[1] = float16v_t{};
    float32v_t smat = float32v_t{};  // "chunk -1": the first chunk's promotion of part[1] adds 0 * 0
    // All first loads are in flight together (one memory latency before the first
    // chunk): the B slice of chunk 0, staged below, then those the loop keeps in
    // flight, in its order (the B slice staged next, the A slice, the B slice
    // after), so the wait counts the compiler derives for the loop body hold on
    // its first pass too.
    {
      Slice b0;
      F::fetch_b(p, t, 0, s1, b0);
      __builtin_amdgcn_sched_barrier(0);
      F::fetch_b(p, t, 1, s1, b1);
      __builtin_amdgcn_sched_barrier(0);
      F::fetch_a(p, t, 0, s1, a);
      __builtin_amdgcn_sched_barrier(0);
      F::fetch_b(p, t, 2, s1, b2);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MIXB) {
        half2_t sg[4];
        FM::prep_b(b0, sg);
        half8_t* out = reinterpret_cast<half8_t*>(sm.b[0] + (threadIdx.x >> 2) * LDS_STRIDE + t.bq * 32);
        out[0] = FM::template unit_b<0>(b0, sg, t.b8);
        out[1] = FM::template unit_b<1>(b0, sg, t.b8);
        out[2] = FM::template unit_b<2>(b0, sg, t.b8);
        out[3] = FM::template unit_b<3>(b0, sg, t.b8);
        sm.sb[0][threadIdx.x >> 2] = b0.S;
      } else {
        stage_first_b<FB0>(sm, t, b0);
      }
    }
    FM::prep_a(a, sga);
    af[0] = FM::template frag_a<0>(a, sga, false);
    barrier_lds();
    constexpr int kFragAhead = kFragAheadSlots;
    half8_t bf[frag_ring(kFragAhead)];
    {
      const _Float16* bb = sm.b[0] + (t.lane & 31) * LDS_STRIDE + (t.lane >> 5) * 64;
      static_for<kFragAhead>([&](auto f) __attribute__((always_inline)) {
        bf[decltype(f)::value] = ld8(bb + decltype(f)::value * 8);
      });
    }
    // Chunk it stages the B slice of chunk it + 1 from b1 (it even) or b2 (it
    // odd) and, once that staging is done (its sync slot), refills the same
    // slice with chunk it + 3.  Two chunks per loop iteration keep the slices
    // in fixed registers, so no copy at the back edge waits on a fresh load.
    auto run = [&](int it, Slice& nb) __attribute__((always_inline)) {
      auto fa = [&](Slice& sl) __attribute__((always_inline)) { F::fetch_a(p, t, it + 1, s1, sl); };
      auto sync = [&]() __attribute__((always_inline)) {
        F::fetch_b(p, t, it + 3, s1, nb);
        barrier_lds();  // chunk it+1's B staged; this chunk's stage may be refilled
      };
      chunk<FM, kFragAhead>(sm, t, it, false, t.b8, af, sga, bf, acc, part, smat, a, nb, fa, sync);
    };
    int it = 0;
    for (; it + 1 < s1; it += 2) {
      run(it, b1);
      run(it + 1, b2);
    }
    if (it < s1) run(it, b1);
    static_for<16>([&](auto e) __attribute__((always_inline)) {
      constexpr int i = decltype(e)::value;
      acc[3][i] = fmaf(part[1][i], smat[16 + i], acc[3][i]);
    });
  }
  if constexpr (FA1 != F_NONE) {
    for (int it = s1; it < n; ++it) tail_chunk<FA1, FB1>(p, sm, t, t.c_begin + it - t.n0c, acc);
  }

  store_tile<MIXB>(p, smem.out, t, m0, n0, z, acc, lo, c1, r0, ncols);
}

// ---------------------------------------------------------------------------
// Image products: B decoded once per product.
//
// Every row tile of the output reads the whole B operand (a 16384-row forward
// reads the weights 64 times), and the kernel above decodes B again in each of
// them (decode, LDS writes and the packed B slices in registers: about a sixth
// of its time).  Here bimage_kernel first decodes B once into f16 chunk images
// laid out exactly as the kernel's LDS stage (128 rows of LDS_STRIDE halfs per
// 128-K chunk and column tile, outlier-column products already in output-column
// order), and gemm_img_kernel copies each image into LDS with
// global_load_lds_dwordx4, which moves the bytes without registers or VALU.
// The cost is one extra pass over B (0.56 B read and 2.1 B written per
// element, small next to the product for weights) and 3.9 times the B bytes
// per tile, served from L2.
static_assert(kImgChunkBytes == BN * LDS_STRIDE * 2 && kImgRowBytes == LDS_STRIDE * 2, "image = LDS stage");
// row tiles from which the image pays for its extra pass (each row tile would
// otherwise decode B again)
constexpr int kImgMinRowTiles = 8;
static_assert(kImgChunkBytes % 1024 == 0 && kImgChunkBytes / 1024 == 34, "image chunk of 34 1 KB blocks");

struct SmemImg {
  _Float16 b[2][BN * LDS_STRIDE];
};

// Tile order of the image products: groups of kImgGroupRows row tiles, rows
// fastest within a group, then the group's next column tile.  A B image is
// 3.8 times the packed bytes and a product's image is larger than an XCD's 4 MB
// L2, so with columns fastest the ~32 tiles an XCD runs at once (its range of
// tile numbers is contiguous) would read the whole image and every row tile
// would fetch it again; in groups, those tiles share 8 row blocks of A and a
// few column tiles of the image.  A bijection of [0, tiles_m * tiles_n) for any
// sizes (the last group may have fewer rows).
constexpr uint32_t kImgGroupRows = 8;
__device__ __forceinline__ void img_tile(uint32_t tile, uint32_t tiles_m, uint32_t tiles_n, uint32_t& tm,
                                         uint32_t& tn) {
  const uint32_t per_group = kImgGroupRows * tiles_n;
  const uint32_t g = tile / per_group, w = tile - g * per_group;
  const uint32_t first = g * kImgGroupRows;
  const uint32_t rows = min(tiles_m - first, kImgGroupRows);
  tm = first + w % rows;
  tn = w / rows;
}
union SmemImgAll {
  SmemImg loop;
  float out[BM / 32][32][OUT_STRIDE];
};

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Copy one chunk image (kImgChunkBytes at src, 16-byte aligned) into the LDS
// stage whose block `w` starts at lds_w, if `on` (wave-uniform): wave w moves
// the 1 KB blocks w, w + 8, w + 16, w + 24 (waves 0 and 1 also w + 32), 16
// bytes per lane (voff = 16 * lane + 1024 * w).  The copy is asynchronous: it
// has landed once this wave's vector-memory counter is zero, and the other
// waves may read it after a barrier that follows that wait.  Written in
// assembly because the compiler's own form makes the next LDS read of any
// stage wait for every outstanding copy (here the chunk's barrier carries the
// wait), and with its two conditions inside the block: a branch around it
// splits the chunk's straight-line code, and the register allocation of the
// chunk then spills.  m0 (the LDS destination) is restored afterwards; the
// first s_nop covers an SGPR operand written by a vector instruction just
// before, the others the m0 write before each copy.
__device__ __forceinline__ void dma_chunk(const uint8_t* src, uint32_t lds_w, uint32_t voff, int w, int on) {
  uint32_t save;
  asm volatile(
      "s_cmp_eq_u32 %[on], 0\n\t"
      "s_cbranch_scc1 2f\n\t"
      "s_mov_b32 %[sv], m0\n\t"
      "s_nop 4\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v], %[b0]\n\t"
      "s_mov_b32 m0, %[m1]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v], %[b1]\n\t"
      "s_mov_b32 m0, %[m2]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v], %[b2]\n\t"
      "s_mov_b32 m0, %[m3]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v], %[b3]\n\t"
      "s_cmp_lt_u32 %[w], 2\n\t"
      "s_cbranch_scc0 1f\n\t"
      "s_mov_b32 m0, %[m4]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v], %[b4]\n"
      "1:\n\t"
      "s_mov_b32 m0, %[sv]\n"
      "2:\n"
      : [sv] "=&s"(save)
      : [on] "s"(__builtin_amdgcn_readfirstlane(on)), [w] "s"(__builtin_amdgcn_readfirstlane(w)), [m0] "s"(lds_w), [m1] "s"(lds_w + 8192u), [m2] "s"(lds_w + 16384u),
        [m3] "s"(lds_w + 24576u), [m4] "s"(lds_w + 32768u), [v] "v"(voff), [b0] "s"(src), [b1] "s"(src + 8192),
        [b2] "s"(src + 16384), [b3] "s"(src + 24576), [b4] "s"(src + 32768)
      : "memory", "scc");
}

// Every outstanding load and LDS access of this wave has completed (the
// stage copies included), then the workgroup barrier.
__device__ __forceinline__ void barrier_all() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

template <int F>
struct FmtTag {
  static constexpr int value = F;
};

// One chunk of an image product: the slots of chunk() above without the B
// staging.  The A fragments come from this chunk's slice `a` (format FA; the
// next chunk's slice `an` is in format FN, which differs from FA only where a
// two-segment product crosses from its NVFP4 to its FP8 segment); at
// slot 7 the next chunk's S_B is requested (fetch_sb) and at slot 8 the slice
// of the chunk after next (fetch_a, into `a`, whose fragments are decoded by
// then); the next chunk's slice `an`, requested one chunk earlier, is prepared
// at slot 30 and its fragment 0 decoded at slot 31.  sync (slot
// 32 - kFragAhead) waits for every load and copy except the slice just
// requested, crosses the barrier (the next stage has landed for all waves,
// this stage is no longer read) and starts the copy of the chunk after next
// into this stage.  sbc holds S_B of this chunk's column pairs (lanes 0-31
// columns of block 2p, lanes 32-63 of block 2p + 1).
template <int FA, int kFragAhead, int FN, class FETCH_SB, class FETCH_A, class SYNC>
__device__ __forceinline__ void chunk_img(const _Float16* bb, const _Float16* bn, half8_t (&af)[8],
                                          half2_t (&sga)[4], half8_t (&bf)[frag_ring(kFragAhead)],
                                          float (&acc)[4][16], float16v_t (&part)[2], float32v_t& smat, Slice& a,
                                          const Slice& an, const float2& sbc, FETCH_SB&& fetch_sb, FETCH_A&& fetch_a,
                                          SYNC&& sync) {
  constexpr int kFragRing = frag_ring(kFragAhead);
  // S_A of this chunk in a register of its own (an opaque copy): the slice's
  // register is refilled at slot 8 while S_A is still needed at slot 24, and
  // without the copy the compiler carries the refilled value into the loop's
  // register with a move at the back edge, which waits for every load in
  // flight (the stage copy included)
  float sa;
  asm volatile("v_mov_b32 %0, %1" : "=v"(sa) : "v"(a.S));
  static_for<32>([&](auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    constexpr int tn = q / 8, ks = q % 8;
    if constexpr (q < 7) af[q + 1] = Op<FA>::template frag_a<q + 1>(a, sga);
    if constexpr (q == 7) fetch_sb();
    if constexpr (q == 8) {
      // the scale products of blocks 0-1 before the slice (and S_A) is refilled
      smat = __builtin_amdgcn_mfma_f32_32x32x1f32(sa, sbc.x, float32v_t{}, 0, 0, 0);
      fetch_a(a);
    }
    if constexpr (q == 30) Op<FN>::prep_a(an, sga);
    if constexpr (q == 31) af[0] = Op<FN>::template frag_a<0>(an, sga);
    if constexpr (q == 32 - kFragAhead) sync();
    constexpr int qf = q + kFragAhead;
    if constexpr (qf < 32) bf[qf % kFragRing] = ld8(bb + (qf / 8) * 32 * LDS_STRIDE + (qf % 8) * 8);
    else bf[qf % kFragRing] = ld8(bn + (qf - 32) * 8);
    if constexpr (q == 24) smat = __builtin_amdgcn_mfma_f32_32x32x1f32(sa, sbc.y, float32v_t{}, 0, 0, 0);
    part[tn & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks], bf[q % kFragRing], ks == 0 ? float16v_t{} : part[tn & 1],
                                                          0, 0, 0);
    if constexpr (ks >= 2) {
      constexpr int pb = tn > 0 ? tn - 1 : 3;
      constexpr int lo = ks <= 6 ? 3 * (ks - 2) : 14, hi = ks < 6 ? lo + 3 : lo + 2;
      static_for<hi - lo>([&](auto i) __attribute__((always_inline)) {
        constexpr int e = lo + decltype(i)::value;
        acc[pb][e] = fmaf(part[pb & 1][e], smat[16 * (pb & 1) + e], acc[pb][e]);
      });
    }
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Workgroup: 512 threads (8 waves), one 256x128 output tile, the chunk range of
// split z; A in format FA (one K segment); B from the chunk images.  Chunk it
// reads stage it & 1; the copy of chunk it + 2 into the same stage starts once
// every wave is past the chunk's barrier.
template <int FA>
__global__ __launch_bounds__(512, 1) void gemm_img_kernel(GemmKArgs p) {
  __shared__ __attribute__((aligned(16))) SmemImgAll smem;
  SmemImg& sm = smem.loop;

  const uint32_t nwg = gridDim.x;
  uint32_t id = blockIdx.x;
  const uint32_t per_xcd = nwg / 8;
  if (id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;
  const uint32_t tiles = (uint32_t)(p.tiles_m * p.tiles_n);
  const uint32_t tile = id % tiles, z = id / tiles;
  uint32_t ti, tj;
  img_tile(tile, (uint32_t)p.tiles_m, (uint32_t)p.tiles_n, ti, tj);
  const int64_t m0 = (int64_t)ti * BM, n0 = (int64_t)tj * BN;

  Ctx t;
  t.lane = threadIdx.x & 63;
  t.w = threadIdx.x >> 6;
  t.ah = t.lane >> 5;
  t.bq = 0;
  t.b8 = false;
  const uint32_t arow = (uint32_t)min(m0 + t.w * 32 + (t.lane & 31), p.I - 1);
  t.arn[0] = t.arn[1] = arow * (uint32_t)p.seg[0].a.ld_s128;
  t.brn[0] = t.brn[1] = 0;
  t.n0c = p.seg[0].nchunks;
  t.c_begin = (int)z * p.chunks_per_split;
  const int n = min(t.c_begin + p.chunks_per_split, p.nchunks) - t.c_begin;

  const uint8_t* img = p.bimg + ((size_t)tj * (size_t)p.nchunks + (size_t)t.c_begin) * kImgChunkBytes;
  const float* sbl = p.bsc + (size_t)t.c_begin * (size_t)p.bsc_ld + n0 + t.lane;
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(lds_addr(sm.b[0]) + (uint32_t)t.w * 1024u);
  const uint32_t voff = (uint32_t)t.lane * 16u + (uint32_t)t.w * 1024u;
  // copy the image of chunk c into stage st if c < n
  auto dma = [&](int c, int st) __attribute__((always_inline)) {
    dma_chunk(img + (size_t)min(c, n - 1) * kImgChunkBytes, lds_w + (uint32_t)st * (uint32_t)kImgChunkBytes, voff,
              t.w, c < n ? 1 : 0);
  };
  auto load_sb = [&](int it, float2& sb) __attribute__((always_inline)) {
    const float* q = sbl + (size_t)min(it, n - 1) * (size_t)p.bsc_ld;
    sb.x = q[0];
    sb.y = q[64];
  };

  float acc[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;

  Slice as[2];
  float2 sbc, sbn;
  // Prologue: chunk 0's A slice, S_B and image; once they have landed, the copy
  // of chunk 1 and the slice of chunk 1 are requested.
  Op<FA>::load_half(p.seg[0].a, t.arn[0], t.c_begin, t.ah, as[0]);
  load_sb(0, sbc);
  dma(0, 0);
  barrier_all();
  dma(1, 1);

  {
    Op<FA>::load_half(p.seg[0].a, t.arn[0], t.c_begin + min(1, n - 1), t.ah, as[1]);
    half8_t af[8];
    half2_t sga[4];
    float16v_t part[2];
    part[1] = float16v_t{};
    float32v_t smat = float32v_t{};  // "chunk -1": the first chunk's promotion of part[1] adds 0 * 0
    constexpr int kFragAhead = kFragAheadSlots;
    half8_t bf[frag_ring(kFragAhead)];
    const int lane_off = (t.lane & 31) * LDS_STRIDE + (t.lane >> 5) * 64;
    Op<FA>::prep_a(as[0], sga);
    af[0] = Op<FA>::template frag_a<0>(as[0], sga);
    {
      const _Float16* bb = sm.b[0] + lane_off;
      static_for<kFragAhead>([&](auto f) __attribute__((always_inline)) {
        bf[decltype(f)::value] = ld8(bb + decltype(f)::value * 8);
      });
    }
    // chunk it in stage ST with slice as[ST] (requests past the range reload
    // the last chunk); S_B alternates between two register pairs.  The barrier's
    // wait leaves only the slice requested at slot 8 in flight (it was issued
    // after the S_B request of slot 7 and after the copy it waits for).
    auto run = [&](auto st, int it) __attribute__((always_inline)) {
      constexpr int ST = decltype(st)::value;
      float2& cur = ST ? sbn : sbc;
      float2& nxt = ST ? sbc : sbn;
      auto fetch_sb = [&]() __attribute__((always_inline)) { load_sb(it + 1, nxt); };
      auto fetch_a = [&](Slice& sl) __attribute__((always_inline)) {
        Op<FA>::load_half(p.seg[0].a, t.arn[0], t.c_begin + min(it + 2, n - 1), t.ah, sl);
      };
      auto sync = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0070 | Op<FA>::kHalfLoads);  // vmcnt(slice loads) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        dma(it + 2, ST);
      };
      chunk_img<FA, kFragAhead, FA>(sm.b[ST] + lane_off, sm.b[ST ^ 1] + lane_off, af, sga, bf, acc, part, smat, as[ST],
                                 as[ST ^ 1], cur, fetch_sb, fetch_a, sync);
    };
    int it = 0;
    for (; it + 1 < n; it += 2) {
      run(FmtTag<0>{}, it);
      run(FmtTag<1>{}, it + 1);
    }
    if (it < n) run(FmtTag<0>{}, it);
    static_for<16>([&](auto e) __attribute__((always_inline)) {
      constexpr int i = decltype(e)::value;
      acc[3][i] = fmaf(part[1][i], smat[16 + i], acc[3][i]);
    });
  }

  store_tile<false>(p, smem.out, t, m0, n0, z, acc, 0, BN, 0, BN);
}

// The forward's two-segment product (NVFP4 x NVFP4 over the rest channels,
// then FP8 x FP8 over the outlier channels) from one chunk image of both
// segments' B rows: the pipelined loop runs through the segment boundary, so
// the FP8 chunks are pipelined like the others.  Each chunk's code knows the
// formats of its own slice, of the next chunk's (decoded at its last slots)
// and of the one it requests (two chunks ahead): NVFP4 up to chunk n0 - 3,
// the crossing at chunks n0 - 2 and n0 - 1, FP8 from n0 on.  P0 = n0 & 1
// fixes the stage parity of the crossing, so stages and slices stay
// compile-time indices.  One split (no K split); n0 >= 2, at least one FP8
// chunk.
template <int P0>
__global__ __launch_bounds__(512, 1) void gemm_img2_kernel(GemmKArgs p) {
  constexpr int N4 = TJ2_NVFP4, F8 = TJ2_FP8;
  __shared__ __attribute__((aligned(16))) SmemImgAll smem;
  SmemImg& sm = smem.loop;

  const uint32_t nwg = gridDim.x;
  uint32_t id = blockIdx.x;
  const uint32_t per_xcd = nwg / 8;
  if (id < per_xcd * 8) id = (id % 8) * per_xcd + id / 8;
  uint32_t ti, tj;
  img_tile(id, (uint32_t)p.tiles_m, (uint32_t)p.tiles_n, ti, tj);
  const int64_t m0 = (int64_t)ti * BM, n0 = (int64_t)tj * BN;

  Ctx t;
  t.lane = threadIdx.x & 63;
  t.w = threadIdx.x >> 6;
  t.ah = t.lane >> 5;
  t.bq = 0;
  t.b8 = false;
  const uint32_t arow = (uint32_t)min(m0 + t.w * 32 + (t.lane & 31), p.I - 1);
  t.arn[0] = arow * (uint32_t)p.seg[0].a.ld_s128;
  t.arn[1] = arow * (uint32_t)p.seg[1].a.ld_s128;
  t.brn[0] = t.brn[1] = 0;
  t.n0c = p.seg[0].nchunks;
  t.c_begin = 0;
  const int n = p.nchunks, nc0 = t.n0c;

  const uint8_t* img = p.bimg + (size_t)tj * (size_t)n * kImgChunkBytes;
  const float* sbl = p.bsc + n0 + t.lane;
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(lds_addr(sm.b[0]) + (uint32_t)t.w * 1024u);
  const uint32_t voff = (uint32_t)t.lane * 16u + (uint32_t)t.w * 1024u;
  auto dma = [&](int c, int st) __attribute__((always_inline)) {
    dma_chunk(img + (size_t)min(c, n - 1) * kImgChunkBytes, lds_w + (uint32_t)st * (uint32_t)kImgChunkBytes, voff,
              t.w, c < n ? 1 : 0);
  };
  auto load_sb = [&](int it, float2& sb) __attribute__((always_inline)) {
    const float* q = sbl + (size_t)min(it, n - 1) * (size_t)p.bsc_ld;
    sb.x = q[0];
    sb.y = q[64];
  };
  // the slice of chunk c in format F (chunks past the range reload the last one)
  auto load_slice = [&](auto ft, int c, Slice& sl) __attribute__((always_inline)) {
    constexpr int F = decltype(ft)::value;
    if constexpr (F == N4) Op<N4>::load_half(p.seg[0].a, t.arn[0], c, t.ah, sl);
    else Op<F8>::load_half(p.seg[1].a, t.arn[1], min(c, n - 1) - nc0, t.ah, sl);
  };

  float acc[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;

  Slice as[2];
  float2 sbc, sbn;
  load_slice(FmtTag<N4>{}, 0, as[0]);
  load_sb(0, sbc);
  dma(0, 0);
  barrier_all();
  dma(1, 1);

  {
    load_slice(FmtTag<N4>{}, 1, as[1]);
    half8_t af[8];
    half2_t sga[4];
    float16v_t part[2];
    part[1] = float16v_t{};
    float32v_t smat = float32v_t{};
    constexpr int kFragAhead = kFragAheadSlots;
    half8_t bf[frag_ring(kFragAhead)];
    const int lane_off = (t.lane & 31) * LDS_STRIDE + (t.lane >> 5) * 64;
    Op<N4>::prep_a(as[0], sga);
    af[0] = Op<N4>::template frag_a<0>(as[0], sga);
    {
      const _Float16* bb = sm.b[0] + lane_off;
      static_for<kFragAhead>([&](auto f) __attribute__((always_inline)) {
        bf[decltype(f)::value] = ld8(bb + decltype(f)::value * 8);
      });
    }
    // chunk it in stage ST: its slice in format FC, the next chunk's in FN, the
    // one requested at slot 8 (chunk it + 2) in FF
    auto run = [&](auto st, auto fc, auto fn, auto ff, int it) __attribute__((always_inline)) {
      constexpr int ST = decltype(st)::value;
      constexpr int FC = decltype(fc)::value, FN = decltype(fn)::value, FF = decltype(ff)::value;
      float2& cur = ST ? sbn : sbc;
      float2& nxt = ST ? sbc : sbn;
      auto fetch_sb = [&]() __attribute__((always_inline)) { load_sb(it + 1, nxt); };
      auto fetch_a = [&](Slice& sl) __attribute__((always_inline)) { load_slice(FmtTag<FF>{}, it + 2, sl); };
      auto sync = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0070 | Op<FF>::kHalfLoads);  // vmcnt(slice loads) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        dma(it + 2, ST);
      };
      chunk_img<FC, kFragAhead, FN>(sm.b[ST] + lane_off, sm.b[ST ^ 1] + lane_off, af, sga, bf, acc, part, smat,
                                    as[ST], as[ST ^ 1], cur, fetch_sb, fetch_a, sync);
    };
    using S0 = FmtTag<0>;
    using S1 = FmtTag<1>;
    using TN = FmtTag<N4>;
    using TF = FmtTag<F8>;
    int it = 0;
    // NVFP4 chunks whose requests are NVFP4 too (it + 2 < n0)
    for (; it + 3 < nc0; it += 2) {
      run(S0{}, TN{}, TN{}, TN{}, it);
      run(S1{}, TN{}, TN{}, TN{}, it + 1);
    }
    if constexpr (P0 == 1) {  // n0 odd: chunk n0 - 3 (stage 0) is the last of them
      run(S0{}, TN{}, TN{}, TN{}, it);
      ++it;
    }
    // the crossing: chunk n0 - 2 requests the first FP8 slice, chunk n0 - 1
    // decodes it at its last slots
    if constexpr (P0 == 0) {
      run(S0{}, TN{}, TN{}, TF{}, it);
      run(S1{}, TN{}, TF{}, TF{}, it + 1);
    } else {
      run(S1{}, TN{}, TN{}, TF{}, it);
      run(S0{}, TN{}, TF{}, TF{}, it + 1);
    }
    it += 2;
    // FP8 chunks, from stage n0 & 1
    if constexpr (P0 == 0) {
      for (; it + 1 < n; it += 2) {
        run(S0{}, TF{}, TF{}, TF{}, it);
        run(S1{}, TF{}, TF{}, TF{}, it + 1);
      }
      if (it < n) run(S0{}, TF{}, TF{}, TF{}, it);
    } else {
      for (; it + 1 < n; it += 2) {
        run(S1{}, TF{}, TF{}, TF{}, it);
        run(S0{}, TF{}, TF{}, TF{}, it + 1);
      }
      if (it < n) run(S1{}, TF{}, TF{}, TF{}, it);
    }
    static_for<16>([&](auto e) __attribute__((always_inline)) {
      constexpr int i = decltype(e)::value;
      acc[3][i] = fmaf(part[1][i], smat[16 + i], acc[3][i]);
    });
  }

  store_tile<false>(p, smem.out, t, m0, n0, 0, acc, 0, BN, 0, BN);
}

// B decode into chunk images: a workgroup of 256 threads per (image chunk, 64
// source rows; a two-segment product's image holds the first segment's chunks,
// then the second's, each chunk decoded from its own segment's B); thread (unit u = t % 16, rows v = 64 * slab + 16k + t / 16,
// k = 0..3) decodes K elements 8u..8u+7 of the chunk in four rows into 16-byte
// pieces of the image (the 16 threads of a row write its 256 bytes; u = 15
// also writes the row's pad, u = 0 its S_B).  Source rows are B's rows in
// order; for outlier-column products rows [0, J - n_outl) are B's NVFP4 rows,
// placed at image row (output column) rest[v], and rows [J - n_outl, J) are
// b8's FP8 rows, placed at outl[v - (J - n_outl)], so every destination is
// known from one load.  Rows J and above of the last column tile are zero.
struct ImgArgs {
  OperandK b;
  int fmt;
  int nchunks;  // chunks of the whole image
  int n0c;      // chunks of the first segment: image chunks from n0c on are the second's (b2, fmt2)
  OperandK b2;
  int fmt2;
  OperandK b8;
  const int32_t* outl;
  const int32_t* rest;
  int n_outl;
  int64_t J, Jpad;
  uint8_t* img;
  float* bsc;
  int64_t bsc_ld;
};

__global__ __launch_bounds__(256) void bimage_kernel(ImgArgs p) {
  const int gi = blockIdx.x;  // image chunk
  const bool seg2 = gi >= p.n0c;  // uniform per workgroup
  const int g = seg2 ? gi - p.n0c : gi;  // chunk of its segment's B
  const OperandK& bop = seg2 ? p.b2 : p.b;
  const int u = threadIdx.x & 15;
  const bool plan = p.outl != nullptr;
  const int64_t nrest = plan ? p.J - p.n_outl : p.J;
  const bool b_fp8 = (seg2 ? p.fmt2 : p.fmt) == TJ2_FP8;
  half8_t f[4];
  float S[4];
  int64_t dest[4];
  // Branch-free: every load is issued for all four rows from addresses chosen
  // per row (a divergent branch would make the compiler wait for each load at
  // its join), then the stores.
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t v = (int64_t)blockIdx.y * 64 + k * 16 + (threadIdx.x >> 4);
    const bool real = v < p.J;
    const bool is8 = plan && real && v >= nrest;                // an FP8 row of b8
    const int64_t r8 = is8 ? v - nrest : 0;
    const int64_t r4 = real && !is8 ? v : 0;
    // the row's destination: loaded for every row from a valid address (without
    // a plan, the first word of B's codes, unused)
    const int32_t* ip = !plan ? reinterpret_cast<const int32_t*>(bop.codes)
                        : is8 ? p.outl + r8 : nrest > 0 ? p.rest + min(v, nrest - 1) : p.outl;
    const int32_t at = *ip;
    dest[k] = plan && real ? (int64_t)at : v;
    const bool fp8 = is8 || b_fp8;
    const size_t rn = is8 ? mul32(r8, p.b8.ld_s128) : mul32(r4, bop.ld_s128);
    const uint8_t* c4 = bop.codes + (size_t)g * 64 + rn * 64 + u * 4;    // NVFP4 codes
    const uint8_t* c8 = (is8 ? p.b8.codes : bop.codes) + (size_t)g * 128 + rn * 128 + u * 8;  // FP8 codes
    const uint8_t* cw = fp8 ? c8 : c4;
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(cw);
    const uint32_t w1 = *reinterpret_cast<const uint32_t*>(fp8 ? cw + 4 : cw);
    const uint32_t sb = *(fp8 ? cw : bop.s16 + (size_t)g * 8 + rn * 8 + (u >> 1));
    const float s128 = ((is8 ? p.b8.s128 : bop.s128) + g)[rn];
    const half2_t s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
    const half8_t v8 = Op<TJ2_FP8>::dec8(w0, w1);
    const half8_t v4 = Op<TJ2_NVFP4>::dec8(w0, half2_t{s2[0], s2[0]});
    f[k] = !real ? half8_t{} : fp8 ? v8 : v4;
    S[k] = real ? s128 : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t d = dest[k];
    if (d < 0 || d >= p.Jpad) continue;  // past the padded rows (or a plan entry out of range)
    uint8_t* dst = p.img + (mul32((uint64_t)d / BN, p.nchunks) + (size_t)gi) * kImgChunkBytes +
                   ((uint64_t)d % BN) * (LDS_STRIDE * 2);
    *reinterpret_cast<half8_t*>(dst + u * 16) = f[k];
    if (u == 0) p.bsc[mul32(gi, p.bsc_ld) + (size_t)d] = S[k];
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

// The common case of the reduction with the split count known at compile time:
// no column map, J and ldc multiples of 4, the output 16-byte aligned.  Every
// partial of the thread's 4 consecutive outputs is requested before the sums
// (taken in split order, as above), and the 4 results leave in one store.
template <int S>
__global__ __launch_bounds__(256) void splitk_reduce4_kernel(const float* __restrict__ partial, int64_t I, int64_t J,
                                                             void* C, int64_t ldc, int c_bf16, int accumulate,
                                                             uint32_t bpr) {
  // bpr workgroups per output row: the row and column come from the workgroup
  // id (one uniform division) instead of a 64-bit division per lane
  const uint32_t i32 = blockIdx.x / bpr;
  const int64_t i = i32;
  const int64_t j0 = ((int64_t)(blockIdx.x - i32 * bpr) * 256 + threadIdx.x) * 4;
  if (j0 >= J) return;
  const int64_t stride = I * J;
  const float* p = partial + i * J + j0;
  float4 v[S];
#pragma unroll
  for (int z = 0; z < S; ++z) v[z] = *reinterpret_cast<const float4*>(p + z * stride);
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
  for (int z = 0; z < S; ++z) {
    s0 += v[z].x; s1 += v[z].y; s2 += v[z].z; s3 += v[z].w;
  }
  if (c_bf16) {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(C) + i * ldc + j0) = make_uint2(pk_bf16(s0, s1), pk_bf16(s2, s3));
  } else {
    float4* cp = reinterpret_cast<float4*>(reinterpret_cast<float*>(C) + i * ldc + j0);
    if (accumulate) {
      const float4 c = *cp;
      *cp = make_float4(c.x + s0, c.y + s1, c.z + s2, c.w + s3);
    } else {
      *cp = make_float4(s0, s1, s2, s3);
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
  if (p.outl) {
    if (p.nseg == 1 && fa == TJ2_NVFP4 && fb == TJ2_NVFP4 && p.b8.fmt == TJ2_FP8)
      return gemm_nt_kernel<TJ2_NVFP4, TJ2_NVFP4, F_NONE, F_NONE, true>;
    if (p.nseg == 1 && fa == TJ2_NVFP6 && fb == TJ2_NVFP4 && p.b8.fmt == TJ2_FP8)
      return gemm_nt_kernel<TJ2_NVFP6, TJ2_NVFP4, F_NONE, F_NONE, true>;
    return nullptr;
  }
  if (p.nseg == 2) {
    if (fa == TJ2_NVFP4 && fb == TJ2_NVFP4 && p.seg[1].a.fmt == TJ2_FP8 && p.seg[1].b.fmt == TJ2_FP8)
      return gemm_nt_kernel<TJ2_NVFP4, TJ2_NVFP4, TJ2_FP8, TJ2_FP8, false>;
    if (fa == TJ2_NVFP4 && fb == TJ2_NVFP4 && p.seg[1].a.fmt == TJ2_NVFP4 && p.seg[1].b.fmt == TJ2_NVFP4)
      return gemm_nt_kernel<TJ2_NVFP4, TJ2_NVFP4, TJ2_NVFP4, TJ2_NVFP4, false>;
    return nullptr;
  }
  if (fa == TJ2_NVFP4 && fb == TJ2_NVFP4) return gemm_nt_kernel<TJ2_NVFP4, TJ2_NVFP4, F_NONE, F_NONE, false>;
  if (fa == TJ2_NVFP6 && fb == TJ2_NVFP4) return gemm_nt_kernel<TJ2_NVFP6, TJ2_NVFP4, F_NONE, F_NONE, false>;
  if (fa == TJ2_NVFP4 && fb == TJ2_FP8) return gemm_nt_kernel<TJ2_NVFP4, TJ2_FP8, F_NONE, F_NONE, false>;
  if (fa == TJ2_FP8 && fb == TJ2_NVFP4) return gemm_nt_kernel<TJ2_FP8, TJ2_NVFP4, F_NONE, F_NONE, false>;
  if (fa == TJ2_FP8 && fb == TJ2_FP8) return gemm_nt_kernel<TJ2_FP8, TJ2_FP8, F_NONE, F_NONE, false>;
  return nullptr;
}

typedef void (*ImgKernel)(GemmKArgs);

ImgKernel pick_img_kernel(const GemmParams& p) {
  if (p.nseg != 1) return nullptr;
  const int fa = p.seg[0].a.fmt, fb = p.seg[0].b.fmt;
  if (fb != TJ2_NVFP4 && fb != TJ2_FP8) return nullptr;
  if (p.outl && (fb != TJ2_NVFP4 || p.b8.fmt != TJ2_FP8)) return nullptr;
  if (fa == TJ2_NVFP4) return gemm_img_kernel<TJ2_NVFP4>;
  if (fa == TJ2_NVFP6) return gemm_img_kernel<TJ2_NVFP6>;
  if (fa == TJ2_FP8) return gemm_img_kernel<TJ2_FP8>;
  return nullptr;
}

}  // namespace

bool gemm_image_pays(int64_t I) { return (I + BM - 1) / BM >= kImgMinRowTiles; }

bool gemm_image_two_segments(const GemmParams& p) {
  return p.nseg == 2 && !p.outl && p.seg[0].a.fmt == TJ2_NVFP4 && p.seg[0].b.fmt == TJ2_NVFP4 &&
         p.seg[1].a.fmt == TJ2_FP8 && p.seg[1].b.fmt == TJ2_FP8 && p.seg[0].K > BK && p.seg[1].K > 0;
}

size_t gemm_image_bytes(int64_t J, int64_t nchunks) {
  const int64_t tn = (J + BN - 1) / BN;
  const size_t img = (size_t)tn * (size_t)nchunks * (size_t)kImgChunkBytes;
  const size_t sc = (size_t)nchunks * (size_t)tn * BN * sizeof(float);
  return img + ((sc + 255) & ~(size_t)255);
}

// K splits of a product: one workgroup per CU at a time (256 CUs).  Estimated
// time in units of one chunk's main loop: rounds of workgroups x (chunks per
// workgroup + kRoundChunks), plus the reduction's HBM traffic for a split
// ((split + 1) fp32 copies of the output, kReduceBytesPerChunk per unit).
// kRoundChunks covers a workgroup's prologue, epilogue and partial tile and
// the loss of a partly filled or repeated round; it is fitted to measured
// products of the weight-gradient shapes (3072x1024, 1024x1024, 4096x1024 and
// 1024x4096 outputs over 16384 tokens), for which it picks the measured best
// split (2, 8, 2, 2).  The smallest split with the least estimated time wins;
// splits keep at least four chunks each.
int gemm_split(int64_t I, int64_t J, int64_t nchunks) {
  constexpr int64_t kCUs = 256;
  constexpr double kRoundChunks = 10.0;
  constexpr double kReduceBytesPerChunk = 12.1e6;
  const int64_t tiles = ((I + BM - 1) / BM) * ((J + BN - 1) / BN);
  if (tiles >= kCUs || nchunks < 8) return 1;
  int64_t best = 1;
  double best_cost = -1.0;
  for (int64_t s = 1; s <= 64 && nchunks / s >= 4; ++s) {
    const int64_t cps = (nchunks + s - 1) / s;
    const int64_t splits = (nchunks + cps - 1) / cps;  // as launched: no empty splits
    if (splits != s) continue;
    const int64_t rounds = (tiles * s + kCUs - 1) / kCUs;
    const double cost = (double)rounds * ((double)cps + kRoundChunks) +
                        (s > 1 ? (double)(s + 1) * (double)I * (double)J * 4.0 / kReduceBytesPerChunk : 0.0);
    if (best_cost < 0.0 || cost < best_cost) { best_cost = cost; best = s; }
  }
  return (int)best;
}

size_t gemm_workspace_bytes(int64_t I, int64_t J, int64_t nchunks) {
  const int split = gemm_split(I, J, nchunks);
  return split > 1 ? (size_t)split * (size_t)I * (size_t)J * sizeof(float) : 0;
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  GemmKernel kern = pick_kernel(p);
  if (!kern) return hipErrorInvalidValue;
  GemmKArgs k;
  k.bimg = nullptr;
  k.bsc = nullptr;
  k.bsc_ld = 0;
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
  k.outl = p.outl;
  k.rest = p.rest;
  k.n_outl = p.n_outl;
  k.b8 = p.outl ? operand_of(p.b8) : k.seg[0].b;
  int split = gemm_split(p.I, p.J, k.nchunks);
  if (split > 1 && (!p.partial || p.partial_bytes < (size_t)split * p.I * p.J * sizeof(float))) split = 1;
  k.chunks_per_split = (k.nchunks + split - 1) / split;
  split = (k.nchunks + k.chunks_per_split - 1) / k.chunks_per_split;  // no empty splits
  k.partial = split > 1 ? p.partial : nullptr;
  k.tiles_m = (int)((p.I + BM - 1) / BM);
  k.tiles_n = (int)((p.J + BN - 1) / BN);
  k.split = split;
  const uint32_t nwg = (uint32_t)k.tiles_m * (uint32_t)k.tiles_n * (uint32_t)split;
  // B is decoded once into chunk images when it is read by many row tiles and
  // the caller gave room for them
  ImgKernel ikern = p.bimg && gemm_image_pays(p.I) ? pick_img_kernel(p) : nullptr;
  if (p.bimg && gemm_image_pays(p.I) && gemm_image_two_segments(p) && split == 1)
    ikern = (k.seg[0].nchunks & 1) ? gemm_img2_kernel<1> : gemm_img2_kernel<0>;
  if (ikern && p.bimg_bytes >= gemm_image_bytes(p.J, k.nchunks) && (reinterpret_cast<uintptr_t>(p.bimg) & 255) == 0) {
    ImgArgs ia;
    ia.b = k.seg[0].b;
    ia.fmt = p.seg[0].b.fmt;
    ia.nchunks = k.nchunks;
    ia.n0c = p.nseg == 2 ? k.seg[0].nchunks : k.nchunks;
    ia.b2 = k.seg[1].b;
    ia.fmt2 = p.nseg == 2 ? p.seg[1].b.fmt : p.seg[0].b.fmt;
    ia.b8 = k.b8;
    ia.outl = p.outl;
    ia.rest = p.rest;
    ia.n_outl = p.n_outl;
    ia.J = p.J;
    ia.Jpad = (int64_t)k.tiles_n * BN;
    ia.img = reinterpret_cast<uint8_t*>(p.bimg);
    ia.bsc_ld = ia.Jpad;
    ia.bsc = reinterpret_cast<float*>(ia.img + (size_t)k.tiles_n * (size_t)k.nchunks * kImgChunkBytes);
    if (!p.bimg_ready) {
      // one decode launch for both segments (a second segment's chunks follow the first's)
      hipLaunchKernelGGL(bimage_kernel, dim3((uint32_t)k.nchunks, (uint32_t)(ia.Jpad / 64)), dim3(256), 0, s, ia);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    k.bimg = ia.img;
    k.bsc = ia.bsc;
    k.bsc_ld = ia.bsc_ld;
    k.outl = nullptr;
    k.rest = nullptr;
    k.n_outl = 0;
    kern = ikern;
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(512), 0, s, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 1) return e;
  const int64_t threads = p.I * ((p.J + 3) / 4);
  const dim3 rgrid((uint32_t)((threads + 255) / 256));
  const int bf = p.c_dtype == TJ2_BF16 ? 1 : 0;
  const int64_t bpr = (p.J / 4 + 255) / 256;  // vector path: workgroups per output row
  const bool vec = !p.col_map && (p.J & 3) == 0 && (p.ldc & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.C) & (bf ? 7 : 15)) == 0 && p.I * bpr < ((int64_t)1 << 31);
  const dim3 vgrid((uint32_t)(p.I * bpr));
  if (vec && split == 2)
    hipLaunchKernelGGL(splitk_reduce4_kernel<2>, vgrid, dim3(256), 0, s, p.partial, p.I, p.J, p.C, p.ldc, bf,
                       p.accumulate, (uint32_t)bpr);
  else if (vec && split == 8)
    hipLaunchKernelGGL(splitk_reduce4_kernel<8>, vgrid, dim3(256), 0, s, p.partial, p.I, p.J, p.C, p.ldc, bf,
                       p.accumulate, (uint32_t)bpr);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel, rgrid, dim3(256), 0, s, p.partial, split, p.I, p.J, p.C, p.ldc,
                       p.col_map, bf, p.accumulate);
  return hipGetLastError();
}

}  // namespace tj2
