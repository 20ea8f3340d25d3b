// libtj2_measure: measurement helpers that bench.py times beside the products.
// They are not part of the path and are built into a library of their own, so
// the product library libtj2 carries none of them (include/tj2_measure.h).
//
// tj2_mfma_peak_probe: the achievable dense f16 MFMA rate of the part.  Each
// wave runs four independent v_mfma_f32_32x32x16_f16 accumulation chains on
// register operands (no memory traffic in the loop), the instruction the
// products use.
//
// tj2_decode_probe: where the B operand of a packed product is decoded.  The
// inner loop of the product kernel without global memory (per 128-K chunk: a
// workgroup barrier, the B stage written to LDS by 512 threads, a second
// barrier, each wave's 8 A fragments decoded in registers, 4 blocks x 8 K
// steps of v_mfma_f32_32x32x16_f16), with B either
//   decoded once per workgroup into f16 in LDS (each thread decodes a quarter
//   row of 32 elements before writing it; waves read 16-byte f16 fragments), or
//   staged packed (E2M1 codes and E4M3 inner scales, 0.5625 B per element) and
//   decoded by every wave after its LDS reads (two 16-byte code reads and one
//   scale word per 32x32 block per lane, then 8 conversions and multiplies per
//   fragment).
// The packed data is synthetic and changes every chunk, so no decode is hoisted
// out of the loop.
//
// tj2_stream_probe: the HBM rate of the OsciReset and master-weight passes'
// access pattern (their loads and stores, no arithmetic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tj2_measure.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float16v_t __attribute__((ext_vector_type(16)));

// 8 E2M1 codes (one word) times an f16 inner scale: 8 exact f16 values
__device__ __forceinline__ half8_t dec8(uint32_t w, half2_t sc) {
  const half2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  const half2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  const half2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  const half2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  return __builtin_bit_cast(half8_t, make_uint4(__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1),
                                                __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3)));
}

// inner scale J (0..3) of a word of four E4M3 codes, as an f16 pair
template <int J>
__device__ __forceinline__ half2_t scale2(uint32_t s4) {
  const half2_t s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s4, 1.0f, J >= 2);
  const _Float16 v = (J & 1) ? s[1] : s[0];
  return half2_t{v, v};
}

constexpr int kPackedPitch = 80;       // bytes per staged packed B row: 64 of codes, 8 of scales, padding
constexpr int kF16Pitch = 128 + 8;     // f16 elements per staged decoded B row

template <bool PACKED>
__global__ __launch_bounds__(512, 1) void decode_probe_kernel(int32_t iters, uint32_t seed, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[PACKED ? 128 * kPackedPitch : 128 * kF16Pitch * 2];
  const int lane = threadIdx.x & 63;
  const int trow = threadIdx.x >> 2, tq = threadIdx.x & 3;  // B staging role: row, quarter
  // synthetic packed data of this thread (codes anywhere on the E2M1 grid, inner scales 2^-2..2^2)
  uint32_t h = seed ^ (threadIdx.x * 0x9E3779B9u) ^ (blockIdx.x * 0x85EBCA6Bu);
  uint32_t aw[8], bw[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) { h = h * 1664525u + 1013904223u; aw[i] = h; }
#pragma unroll
  for (int i = 0; i < 4; ++i) { h = h * 1664525u + 1013904223u; bw[i] = h; }
  const uint32_t sc_word = 0x38383838u ^ ((h >> 8) & 0x07070707u);
  float16v_t acc[4] = {};
  for (int32_t it = 0; it < iters; ++it) {
    const uint32_t x = (uint32_t)it * 0x9E3779B9u;
    __syncthreads();  // every wave is done with the previous chunk's stage
    if (PACKED) {
      *reinterpret_cast<uint4*>(lds + trow * kPackedPitch + tq * 16) =
          make_uint4(bw[0] ^ x, bw[1] ^ x, bw[2] ^ x, bw[3] ^ x);
      if (tq < 2) *reinterpret_cast<uint32_t*>(lds + trow * kPackedPitch + 64 + tq * 4) = sc_word ^ (x & 0x01010101u);
    } else {
      const uint32_t s4 = sc_word ^ (x & 0x01010101u);
      half8_t* dst = reinterpret_cast<half8_t*>(lds + (trow * kF16Pitch + tq * 32) * 2);
      // the quarter's two inner scales (the row's groups 2 tq and 2 tq + 1)
      const half2_t s0 = (tq & 1) ? scale2<2>(s4) : scale2<0>(s4), s1 = (tq & 1) ? scale2<3>(s4) : scale2<1>(s4);
      dst[0] = dec8(bw[0] ^ x, s0);
      dst[1] = dec8(bw[1] ^ x, s0);
      dst[2] = dec8(bw[2] ^ x, s1);
      dst[3] = dec8(bw[3] ^ x, s1);
    }
    __syncthreads();
    // this lane's 8 A fragments (K half lane >> 5 of its row), decoded in registers
    half8_t af[8];
    const uint32_t as = sc_word ^ (x & 0x01010101u);
    const half2_t sa[4] = {scale2<0>(as), scale2<1>(as), scale2<2>(as), scale2<3>(as)};
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = dec8(aw[i] ^ x, sa[i >> 1]);
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const int row = tn * 32 + (lane & 31);
      if (PACKED) {
        const uint8_t* rp = lds + row * kPackedPitch;
        const uint4 c0 = *reinterpret_cast<const uint4*>(rp + (lane >> 5) * 32);
        const uint4 c1 = *reinterpret_cast<const uint4*>(rp + (lane >> 5) * 32 + 16);
        const uint32_t s4 = *reinterpret_cast<const uint32_t*>(rp + 64 + (lane >> 5) * 4);
        const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const half2_t sb[4] = {scale2<0>(s4), scale2<1>(s4), scale2<2>(s4), scale2<3>(s4)};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          acc[tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks], dec8(cw[ks], sb[ks >> 1]), acc[tn], 0, 0, 0);
      } else {
        const _Float16* rp = reinterpret_cast<const _Float16*>(lds) + row * kF16Pitch + (lane >> 5) * 64;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          acc[tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks], *reinterpret_cast<const half8_t*>(rp + ks * 8),
                                                           acc[tn], 0, 0, 0);
      }
    }
  }
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = ((acc[0][0] + acc[1][0]) + acc[2][0]) + acc[3][0];
}

__global__ __launch_bounds__(256) void mfma_peak_kernel(int32_t iters, _Float16 x, float* __restrict__ out) {
  const half8_t a = {x, x, x, x, x, x, x, x};
  float16v_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int32_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c3, 0, 0, 0);
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = ((c0[0] + c1[0]) + c2[0]) + c3[0];
}

// The access pattern of the OsciReset pass (NS = 5 reads, ND = 4 writes) and of
// the fused master pass (7 reads, 6 writes) without their arithmetic: lane g
// owns elements 8g..8g+7 of every array (two 16-byte pieces), issues all its
// loads, then writes dst[i] = src[i] + src[NS - 1].
struct StreamArgs {
  const float* src[8];
  float* dst[8];
  int64_t n8;
};

template <int NS, int ND>
__global__ __launch_bounds__(256) void stream_probe_kernel(StreamArgs a) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= a.n8) return;
  float4 x[NS][2];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const float4* q = reinterpret_cast<const float4*>(a.src[i] + g * 8);
    x[i][0] = q[0];
    x[i][1] = q[1];
  }
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    float4* q = reinterpret_cast<float4*>(a.dst[i] + g * 8);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 u = x[i][h], v = x[NS - 1][h];
      q[h] = make_float4(u.x + v.x, u.y + v.y, u.z + v.z, u.w + v.w);
    }
  }
}

}  // namespace

extern "C" int32_t tj2_stream_probe(const float* const* src, int32_t nsrc, float* const* dst, int32_t ndst, int64_t n,
                                    void* stream) {
  if (!src || !dst || n < 8 || n > ((int64_t)1 << 36) || !((nsrc == 5 && ndst == 4) || (nsrc == 7 && ndst == 6)))
    return 1;
  StreamArgs a{};
  for (int i = 0; i < nsrc; ++i) {
    if (!src[i] || (reinterpret_cast<uintptr_t>(src[i]) & 15u)) return 1;
    a.src[i] = src[i];
  }
  for (int i = 0; i < ndst; ++i) {
    if (!dst[i] || (reinterpret_cast<uintptr_t>(dst[i]) & 15u)) return 1;
    a.dst[i] = dst[i];
  }
  a.n8 = n / 8;
  const dim3 grid((uint32_t)((a.n8 + 255) / 256));
  if (nsrc == 5)
    hipLaunchKernelGGL((stream_probe_kernel<5, 4>), grid, dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((stream_probe_kernel<7, 6>), grid, dim3(256), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int32_t tj2_decode_probe(int32_t packed_b, int64_t workgroups, int32_t iters, float* out, void* stream) {
  if (!out || workgroups < 1 || workgroups > ((int64_t)1 << 20) || iters < 1 || iters > (1 << 20)) return 1;
  if (packed_b)
    hipLaunchKernelGGL(decode_probe_kernel<true>, dim3((uint32_t)workgroups), dim3(512), 0, (hipStream_t)stream,
                       iters, 0x1234567u, out);
  else
    hipLaunchKernelGGL(decode_probe_kernel<false>, dim3((uint32_t)workgroups), dim3(512), 0, (hipStream_t)stream,
                       iters, 0x1234567u, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int32_t tj2_mfma_peak_probe(int64_t workgroups, int32_t iters, float* out, void* stream) {
  if (!out || workgroups < 1 || workgroups > ((int64_t)1 << 20) || iters < 1 || iters > (1 << 20)) return 1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((uint32_t)workgroups), dim3(256), 0, (hipStream_t)stream, iters,
                     (_Float16)0.0625f, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
