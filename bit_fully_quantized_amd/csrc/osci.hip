// OsciReset state update and OutControl calibration helper for gfx950.
//
// OsciReset (TetraJet-v2 technical summary, section 2.B): per weight element,
// the distance travelled by the quantized weight (dQ) and by the master
// weight (dM) are accumulated over a window; at the window end, elements whose
// risk dQ / dM exceeds tau (while the learning rate is low: host switch) are
// reset to the centre of their current bin, Q(w).  Q is the forward quantizer
// (round to nearest, 1x16 groups along K), so the pass also emits the codes the
// next forward consumes.  One lane owns 16 consecutive elements of a row; the 8
// lanes of a 128-element outer block reduce its amax with DPP.  The pass is
// element-wise and HBM-bound: 5 fp32 reads, 4-5 fp32 writes per element.
//
// Calibration (section 2.C): per-channel sum of squares of the activations.
#include "tj2_device.h"
#include "tj2_internal.h"

namespace tj2 {

namespace {

__device__ __forceinline__ void load16f(const float* p, float v[16]) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4 a = q[i];
    v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
  }
}

__device__ __forceinline__ void store16f(float* p, const float v[16]) {
  float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// Forward quantization of one 16-element group: codes and dequantized values.
__device__ __forceinline__ void fwd_quant16(const float w[16], bool valid, uint32_t codes[2], uint32_t* s_code,
                                            float* S, float q[16]) {
  float a_j = 0.0f;
#pragma unroll
  for (int t = 0; t < 16; ++t) a_j = fmaxf(a_j, fabsf(w[t]));
  if (!valid) a_j = 0.0f;
  const float a_o = max8_lanes(a_j);
  GroupScale g = nvfp4_group_scale(a_o, a_j);
  const float s = e4m3_decode(g.s_code);
  float y[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) y[t] = (valid ? w[t] : 0.0f) * g.inv;
  e2m1_rtn16(y, codes);
  typedef float float2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int b = 0; b < 8; ++b) {  // byte b holds elements 2b, 2b+1; exact E2M1 values
    const uint32_t word = codes[b >> 2];
    const float2_t v = (b & 3) == 0   ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0)
                       : (b & 3) == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1)
                       : (b & 3) == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2)
                                      : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
    q[2 * b] = (v.x * s) * g.S;
    q[2 * b + 1] = (v.y * s) * g.S;
  }
  *s_code = g.s_code;
  *S = g.S;
}

__global__ __launch_bounds__(256) void osci_kernel(OsciParams p, int32_t groups_per_row) {
  const uint32_t g = blockIdx.x * 256u + threadIdx.x;
  const uint32_t row = g / (uint32_t)groups_per_row;
  if (row >= (uint32_t)p.N) return;  // whole outer blocks exit together
  const uint32_t j = g - row * (uint32_t)groups_per_row;
  const bool valid = (int64_t)j * 16 < p.K;
  const int64_t base = (int64_t)row * p.K + (int64_t)j * 16;

  // every load of the lane is issued before the quantization work (few waves per
  // SIMD for these sizes, so one exposed latency instead of two)
  float w[16], q[16], wp[16], qp[16], dq[16], dm[16];
  if (valid) {
    load16f(p.W + base, w);
    if (p.mode != TJ2_OSCI_INIT) {
      load16f(p.W_prev + base, wp);
      load16f(p.Q_prev + base, qp);
      load16f(p.dQ + base, dq);
      load16f(p.dM + base, dm);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) w[t] = 0.0f;
  }
  uint32_t codes[2], s_code;
  float S;
  fwd_quant16(w, valid, codes, &s_code, &S, q);

  uint32_t n_reset = 0;
  bool any_reset = false;
  if (valid) {
    if (p.mode == TJ2_OSCI_INIT) {
      float z[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) z[t] = 0.0f;
      store16f(p.W_prev + base, w);
      store16f(p.Q_prev + base, q);
      store16f(p.dQ + base, z);
      store16f(p.dM + base, z);
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        dq[t] = dq[t] + fabsf(q[t] - qp[t]);
        dm[t] = dm[t] + fabsf(w[t] - wp[t]);
        wp[t] = w[t];
      }
      if (p.mode == TJ2_OSCI_WINDOW_END) {
        if (p.reset_enabled) {
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            if (dq[t] > p.tau * dm[t]) {
              w[t] = q[t];
              wp[t] = q[t];
              ++n_reset;
            }
          }
          if (n_reset) store16f(p.W + base, w);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) { dq[t] = 0.0f; dm[t] = 0.0f; }
      }
      store16f(p.W_prev + base, wp);
      store16f(p.Q_prev + base, q);
      store16f(p.dQ + base, dq);
      store16f(p.dM + base, dm);
    }
  }
  any_reset = max8_lanes(n_reset ? 1.0f : 0.0f) > 0.0f;
  if (p.have_wq) {
    if (any_reset) fwd_quant16(w, valid, codes, &s_code, &S, q);  // scales may change after a reset
    const QView& o = p.wq;
    *reinterpret_cast<uint2*>(o.codes + (int64_t)row * o.ld_codes + j * 8u) = make_uint2(codes[0], codes[1]);
    o.s16[(int64_t)row * o.ld_s16 + j] = (uint8_t)s_code;
    if ((j & 7u) == 0u) o.s128[(int64_t)row * o.ld_s128 + (j >> 3)] = S;
  }
  if (p.reset_count && n_reset) atomicAdd(p.reset_count, (unsigned long long)n_reset);
}

// acc[k] += sum_m X[m, k]^2.  Thread: 8 columns x 64 rows; 8 row slices per block
// are reduced in LDS, then one atomic per column per block.
__global__ __launch_bounds__(256) void sumsq_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                    float* __restrict__ acc) {
  __shared__ float red[8][256];
  const int cgp = threadIdx.x & 31, slice = threadIdx.x >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * 256 + cgp * 8;
  const int64_t rbeg = (int64_t)blockIdx.y * 512 + slice * 64;
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c0 < K) {
    for (int r = 0; r < 64; ++r) {
      const int64_t row = rbeg + r;
      if (row >= M) break;
      uint4 a = *reinterpret_cast<const uint4*>(X + row * K + c0);
      uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
        s[2 * i] = fmaf(lo, lo, s[2 * i]);
        s[2 * i + 1] = fmaf(hi, hi, s[2 * i + 1]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[slice][cgp * 8 + i] = s[i];
  __syncthreads();
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col < K) {
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += red[i][threadIdx.x];
    atomicAdd(acc + col, t);
  }
}

}  // namespace

hipError_t launch_osci(const OsciParams& p, hipStream_t s) {
  const int64_t nb = (p.K + 127) / 128;
  const int64_t gpr = nb * 8;
  const int64_t blocks = (p.N * gpr + 255) / 256;
  hipLaunchKernelGGL(osci_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, p, (int32_t)gpr);
  return hipGetLastError();
}

hipError_t launch_channel_sumsq(const void* X, int64_t M, int64_t K, float* acc, hipStream_t s) {
  dim3 grid((uint32_t)((K + 255) / 256), (uint32_t)((M + 511) / 512));
  hipLaunchKernelGGL(sumsq_kernel, grid, dim3(256), 0, s, reinterpret_cast<const uint16_t*>(X), M, K, acc);
  return hipGetLastError();
}

}  // namespace tj2
