// OsciReset state update and OutControl calibration helper for gfx950.
//
// OsciReset (TetraJet-v2 technical summary, section 2.B): per weight element,
// the distance travelled by the quantized weight (dQ) and by the master
// weight (dM) are accumulated over a window; at the window end, elements whose
// risk dQ / dM exceeds tau (while the learning rate is low: host switch) are
// reset to the centre of their current bin, Q(w).  Q is the forward quantizer
// (round to nearest, 1x16 groups along K), so the pass also emits the codes the
// next forward consumes.  One lane owns 8 consecutive elements of a row (half
// a 16-element group); the 16 lanes of a 128-element outer block reduce its
// amax with DPP.  The pass is element-wise and HBM-bound: 5 fp32 reads, 4-5
// fp32 writes per element.
//
// Oscillation diagnostics (section 1 names the phenomenon: quantized weights
// flipping between adjacent bins under small master updates): per call, the
// number of elements whose E2M1 code differs from the previous master's (the
// previous master is quantized once more for it), and at a window end the histogram of
// the window's risk dQ / dM, reduced per workgroup in LDS and added to device
// counters with one atomic per workgroup and counter.
//
// Calibration (section 2.C): per-channel sum of squares of the activations, in
// fp64 and a fixed summation order (two passes, no atomics).
#include <cstring>

#include "tj2_device.h"
#include "tj2_internal.h"

namespace tj2 {

namespace {

__device__ __forceinline__ void load8f(const float* p, float v[8]) {
  const float4* q = reinterpret_cast<const float4*>(p);
  const float4 a = q[0], b = q[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void store8f(float* p, const float v[8]) {
  float4* q = reinterpret_cast<float4*>(p);
  q[0] = make_float4(v[0], v[1], v[2], v[3]);
  q[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// Max over the 16 consecutive lanes of an aligned outer block (non-negative
// inputs: their fp32 bit patterns order as unsigned integers).
__device__ __forceinline__ float max16_lanes(float x) {
  uint32_t xi = __float_as_uint(x);
  xi = max(xi, (uint32_t)__builtin_amdgcn_mov_dpp((int)xi, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  xi = max(xi, (uint32_t)__builtin_amdgcn_mov_dpp((int)xi, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  xi = max(xi, (uint32_t)__builtin_amdgcn_mov_dpp((int)xi, 0x141, 0xF, 0xF, false));  // row_half_mirror
  xi = max(xi, (uint32_t)__builtin_amdgcn_mov_dpp((int)xi, 0x140, 0xF, 0xF, false));  // row_mirror
  return __uint_as_float(xi);
}

// Forward quantization of this lane's half (8 elements) of a 16-element group:
// the group's amax pairs the two lanes, the outer block's spans 16 lanes.
// Returns the lane's 8 codes (one word), the group's E4M3 code and S, and the
// dequantized values Q(w).
__device__ __forceinline__ void fwd_quant8(const float w[8], bool valid, uint32_t* code, uint32_t* s_code, float* S,
                                           float q[8]) {
  float a_h = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) a_h = fmaxf(a_h, fabsf(w[t]));
  if (!valid) a_h = 0.0f;
  uint32_t ai = __float_as_uint(a_h);
  ai = max(ai, (uint32_t)__builtin_amdgcn_mov_dpp((int)ai, 0xB1, 0xF, 0xF, false));  // the group's other half
  const float a_j = __uint_as_float(ai);
  const float a_o = max16_lanes(a_j);
  GroupScale g = nvfp4_group_scale(a_o, a_j);
  const float s = e4m3_decode(g.s_code);
  float y[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) y[t] = (valid ? w[t] : 0.0f) * g.inv;
  uint32_t c = 0u;
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, y[0], y[1], 1.0f, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, y[2], y[3], 1.0f, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, y[4], y[5], 1.0f, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, y[6], y[7], 1.0f, 3);
  typedef float float2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int b = 0; b < 4; ++b) {  // byte b holds elements 2b, 2b+1; exact E2M1 values
    const float2_t v = b == 0   ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0)
                       : b == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1)
                       : b == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2)
                                : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
    q[2 * b] = (v.x * s) * g.S;
    q[2 * b + 1] = (v.y * s) * g.S;
  }
  *code = c;
  *s_code = g.s_code;
  *S = g.S;
}

// Risk bin of one element from its window distances: 0 if dq == 0, 31 if only
// dm == 0, else the binary exponent e of r = dq / dm (fp32, correctly rounded)
// as min(max(e + 16, 1), 30).
__device__ __forceinline__ uint32_t risk_bin(float dq, float dm) {
  if (dq == 0.0f) return 0u;
  if (dm == 0.0f) return (uint32_t)(kRiskBins - 1);
  const float r = dq / dm;
  const int e = (int)((__float_as_uint(r) >> 23) & 0xFFu) - 127;
  return (uint32_t)min(max(e + 16, 1), kRiskBins - 2);
}

// Bin changes between two words of 8 E2M1 codes (sign bit 3 of each nibble);
// +0 and -0 are one bin.
__device__ __forceinline__ uint32_t code_flips(uint32_t c, uint32_t cp) {
  uint32_t n = 0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t a = (c >> (4 * t)) & 15u, b = (cp >> (4 * t)) & 15u;
    n += (a != b && ((a | b) & 7u) != 0u) ? 1u : 0u;
  }
  return n;
}

struct DiagSmem {
  uint32_t flips;
  uint32_t hist[kRiskBins];
};

// Adds the workgroup's flip count and (with bins) risk histogram to the device
// counters.  Called by every thread of the workgroup under a condition that is
// uniform over the grid (kernel parameters), so the barriers are reached by all.
__device__ __forceinline__ void add_diag(DiagSmem& sm, unsigned long long* flips, unsigned long long* hist,
                                         uint32_t n_flip, bool with_bins, const uint32_t (&bins)[8]) {
  if (threadIdx.x == 0) sm.flips = 0u;
  if (threadIdx.x < kRiskBins) sm.hist[threadIdx.x] = 0u;
  __syncthreads();
  if (n_flip) atomicAdd(&sm.flips, n_flip);
  if (with_bins) {
#pragma unroll
    for (int t = 0; t < 8; ++t) atomicAdd(&sm.hist[bins[t]], 1u);
  }
  __syncthreads();
  if (flips && threadIdx.x == 0 && sm.flips) atomicAdd(flips, (unsigned long long)sm.flips);
  if (hist && threadIdx.x < kRiskBins && sm.hist[threadIdx.x])
    atomicAdd(hist + threadIdx.x, (unsigned long long)sm.hist[threadIdx.x]);
}

// One lane per half group (8 consecutive elements of a row); the 16 lanes of
// a 128-element outer block are consecutive.  All loads of the lane are issued
// before the quantization work.  Lanes past the last row stay (no early exit,
// the diagnostics use workgroup barriers) but touch no memory.
template <bool DIAG>
__device__ __forceinline__ void osci_body(const OsciParams& p, int32_t halves_per_row, uint32_t g, DiagSmem& dsm) {
  const uint32_t row = g / (uint32_t)halves_per_row;
  const bool live = row < (uint32_t)p.N;  // whole outer blocks are live or not
  const uint32_t jh = g - row * (uint32_t)halves_per_row;
  const uint32_t j = jh >> 1;  // 16-element group
  const bool valid = live && (int64_t)j * 16 < p.K;
  const int64_t base = (int64_t)row * p.K + (int64_t)jh * 8;

  float w[8], q[8], wp[8], qp[8], dq[8], dm[8];
  if (valid) {
    load8f(p.W + base, w);
    if (p.mode != TJ2_OSCI_INIT) {
      load8f(p.W_prev + base, wp);
      load8f(p.Q_prev + base, qp);
      load8f(p.dQ + base, dq);
      load8f(p.dM + base, dm);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) w[t] = 0.0f;
  }
  uint32_t code, s_code;
  float S;
  fwd_quant8(w, valid, &code, &s_code, &S, q);
  uint32_t code_prev = 0;  // diagnostics: the previous master's codes (a flip is a change of bin)
  if (DIAG && p.mode != TJ2_OSCI_INIT) {
    float x[8], qx[8], Sx;
    uint32_t sx;
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = valid ? wp[t] : 0.0f;
    fwd_quant8(x, valid, &code_prev, &sx, &Sx, qx);
  }

  uint32_t n_reset = 0, n_flip = 0;
  uint32_t bins[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const bool want_bins = DIAG && p.risk_hist && p.mode == TJ2_OSCI_WINDOW_END;
  if (valid) {
    if (p.mode == TJ2_OSCI_INIT) {
      float z[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) z[t] = 0.0f;
      store8f(p.W_prev + base, w);
      store8f(p.Q_prev + base, q);
      store8f(p.dQ + base, z);
      store8f(p.dM + base, z);
    } else {
      if (DIAG) n_flip = code_flips(code, code_prev);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        dq[t] = dq[t] + fabsf(q[t] - qp[t]);
        dm[t] = dm[t] + fabsf(w[t] - wp[t]);
        wp[t] = w[t];
      }
      if (p.mode == TJ2_OSCI_WINDOW_END) {
        if (want_bins) {
#pragma unroll
          for (int t = 0; t < 8; ++t) bins[t] = risk_bin(dq[t], dm[t]);
        }
        if (p.reset_enabled) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            if (dq[t] > p.tau * dm[t]) {
              w[t] = q[t];
              wp[t] = q[t];
              ++n_reset;
            }
          }
          if (n_reset) store8f(p.W + base, w);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) { dq[t] = 0.0f; dm[t] = 0.0f; }
      }
      store8f(p.W_prev + base, wp);
      store8f(p.Q_prev + base, q);
      store8f(p.dQ + base, dq);
      store8f(p.dM + base, dm);
    }
  }
  const bool any_reset = max16_lanes(n_reset ? 1.0f : 0.0f) > 0.0f;  // uniform over the outer block
  if (p.have_wq && live) {
    if (any_reset) fwd_quant8(w, valid, &code, &s_code, &S, q);  // scales may change after a reset
    const QView& o = p.wq;
    *reinterpret_cast<uint32_t*>(o.codes + (int64_t)row * o.ld_codes + jh * 4u) = code;
    if ((jh & 1u) == 0u) o.s16[(int64_t)row * o.ld_s16 + j] = (uint8_t)s_code;
    if ((jh & 15u) == 0u) o.s128[(int64_t)row * o.ld_s128 + (j >> 3)] = S;
  }
  if (p.reset_count && n_reset) atomicAdd(p.reset_count, (unsigned long long)n_reset);
  if constexpr (DIAG) add_diag(dsm, p.flips, want_bins ? p.risk_hist : nullptr, n_flip, want_bins && valid, bins);
}

template <bool DIAG>
__global__ __launch_bounds__(256) void osci_kernel(OsciParams p, int32_t halves_per_row) {
  __shared__ DiagSmem dsm;
  osci_body<DIAG>(p, halves_per_row, blockIdx.x * 256u + threadIdx.x, dsm);
}

// Several problems per launch (a model's weight matrices after one optimizer
// step), so that small matrices do not each pay a launch.
struct OsciMulti {
  OsciParams p[kOsciMultiMax];
  uint32_t begin[kOsciMultiMax + 1];
  int32_t hpr[kOsciMultiMax];
  int n;
};
static_assert(sizeof(OsciMulti) <= 4096, "kernel arguments stay within 4 KB");

template <bool DIAG>
__global__ __launch_bounds__(256) void osci_multi_kernel(OsciMulti m) {
  __shared__ DiagSmem dsm;
  int i = 0;
  while (i + 1 < m.n && blockIdx.x >= m.begin[i + 1]) ++i;  // uniform per workgroup
  osci_body<DIAG>(m.p[i], m.hpr[i], (blockIdx.x - m.begin[i]) * 256u + threadIdx.x, dsm);
}

// Fused master-weight pass (one read of the masters, their AdamW moments and the
// OsciReset state): AdamW with decoupled weight decay in fp32, one rounded
// operation at a time (the builder's optimizer: the pages use fp32 masters and
// apply OsciReset after the update, section 2.B, without naming the optimizer),
// then the OsciReset update of the new masters with the pre-update master as
// W_prev (the distance the master travels is the update), then the forward
// codes.  Lane layout as osci_kernel.
template <bool DIAG>
__device__ __forceinline__ void master_body(const MasterParams& p, int32_t halves_per_row, uint32_t g,
                                            DiagSmem& dsm) {
  const uint32_t row = g / (uint32_t)halves_per_row;
  const bool live = row < (uint32_t)p.N;  // as osci_kernel: no early exit
  const uint32_t jh = g - row * (uint32_t)halves_per_row;
  const uint32_t j = jh >> 1;
  const bool valid = live && (int64_t)j * 16 < p.K;
  const int64_t base = (int64_t)row * p.K + (int64_t)jh * 8;

  float w[8], m[8], v[8], gr[8], qp[8], dq[8], dm[8];
  if (valid) {
    load8f(p.W + base, w);
    load8f(p.m + base, m);
    load8f(p.v + base, v);
    load8f(p.grad + base, gr);
    load8f(p.Q_prev + base, qp);
    load8f(p.dQ + base, dq);
    load8f(p.dM + base, dm);
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) w[t] = 0.0f;
  }
  const float omb1 = 1.0f - p.beta1, omb2 = 1.0f - p.beta2;
  const float decay = 1.0f - p.lr * p.weight_decay;
  float w1[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float m1 = p.beta1 * m[t] + omb1 * gr[t];
    const float v1 = p.beta2 * v[t] + omb2 * (gr[t] * gr[t]);
    const float u = (m1 / p.bc1) / (sqrtf(v1 / p.bc2) + p.eps);
    w1[t] = valid ? w[t] * decay - p.lr * u : 0.0f;
    m[t] = m1;
    v[t] = v1;
  }
  uint32_t code, s_code;
  float S;
  float q[8];
  fwd_quant8(w1, valid, &code, &s_code, &S, q);
  uint32_t code_prev = 0;  // diagnostics: codes of the pre-update master
  if (DIAG) {
    float qx[8], Sx;
    uint32_t sx;
    fwd_quant8(w, valid, &code_prev, &sx, &Sx, qx);
  }
  uint32_t n_reset = 0, n_flip = 0;
  uint32_t bins[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const bool want_bins = DIAG && p.risk_hist && p.window_end;
  if (valid) {
    if (DIAG) n_flip = code_flips(code, code_prev);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      dq[t] = dq[t] + fabsf(q[t] - qp[t]);
      dm[t] = dm[t] + fabsf(w1[t] - w[t]);
    }
    if (p.window_end) {
      if (want_bins) {
#pragma unroll
        for (int t = 0; t < 8; ++t) bins[t] = risk_bin(dq[t], dm[t]);
      }
      if (p.reset_enabled) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if (dq[t] > p.tau * dm[t]) {
            w1[t] = q[t];
            ++n_reset;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) { dq[t] = 0.0f; dm[t] = 0.0f; }
    }
    store8f(p.W + base, w1);
    store8f(p.m + base, m);
    store8f(p.v + base, v);
    store8f(p.Q_prev + base, q);
    store8f(p.dQ + base, dq);
    store8f(p.dM + base, dm);
  }
  const bool any_reset = max16_lanes(n_reset ? 1.0f : 0.0f) > 0.0f;  // uniform over the outer block
  if (p.have_wq && live) {
    if (any_reset) fwd_quant8(w1, valid, &code, &s_code, &S, q);  // scales may change after a reset
    const QView& o = p.wq;
    *reinterpret_cast<uint32_t*>(o.codes + (int64_t)row * o.ld_codes + jh * 4u) = code;
    if ((jh & 1u) == 0u) o.s16[(int64_t)row * o.ld_s16 + j] = (uint8_t)s_code;
    if ((jh & 15u) == 0u) o.s128[(int64_t)row * o.ld_s128 + (j >> 3)] = S;
  }
  if (p.reset_count && n_reset) atomicAdd(p.reset_count, (unsigned long long)n_reset);
  if constexpr (DIAG) add_diag(dsm, p.flips, want_bins ? p.risk_hist : nullptr, n_flip, want_bins && valid, bins);
}

template <bool DIAG>
__global__ __launch_bounds__(256) void master_kernel(MasterParams p, int32_t halves_per_row) {
  __shared__ DiagSmem dsm;
  master_body<DIAG>(p, halves_per_row, blockIdx.x * 256u + threadIdx.x, dsm);
}

// Several weight matrices per launch, as osci_multi_kernel.
struct MasterMulti {
  MasterParams p[kOsciMultiMax];
  uint32_t begin[kOsciMultiMax + 1];
  int32_t hpr[kOsciMultiMax];
  int n;
};
static_assert(sizeof(MasterMulti) <= 4096, "kernel arguments stay within 4 KB");

template <bool DIAG>
__global__ __launch_bounds__(256) void master_multi_kernel(MasterMulti m) {
  __shared__ DiagSmem dsm;
  int i = 0;
  while (i + 1 < m.n && blockIdx.x >= m.begin[i + 1]) ++i;  // uniform per workgroup
  master_body<DIAG>(m.p[i], m.hpr[i], (blockIdx.x - m.begin[i]) * 256u + threadIdx.x, dsm);
}

// Per-channel sums of squares, in a fixed order so that the result does not
// depend on scheduling: kSumsqRows-row slabs of a 256-column tile, each thread 8
// columns x kSumsqRows/8 rows, squares and sums in fp64 (a bf16 square is exact
// in fp64); the 8 row slices of a slab are added in LDS in slice order and the
// slab's sums written to partial[slab][k].
__global__ __launch_bounds__(256) void sumsq_partial_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                            double* __restrict__ partial) {
  __shared__ double red[8][256];
  const int cgp = threadIdx.x & 31, slice = threadIdx.x >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * 256 + cgp * 8;
  constexpr int kRowsPerSlice = kSumsqRows / 8;
  const int64_t rbeg = (int64_t)blockIdx.y * kSumsqRows + slice * kRowsPerSlice;
  double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c0 < K) {
    for (int r = 0; r < kRowsPerSlice; ++r) {
      const int64_t row = rbeg + r;
      if (row >= M) break;
      const uint4 a = *reinterpret_cast<const uint4*>(X + row * K + c0);
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double lo = (double)__uint_as_float(w[i] << 16), hi = (double)__uint_as_float(w[i] & 0xFFFF0000u);
        s[2 * i] = s[2 * i] + lo * lo;
        s[2 * i + 1] = s[2 * i + 1] + hi * hi;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[slice][cgp * 8 + i] = s[i];
  __syncthreads();
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col < K) {
    double t = red[0][threadIdx.x];
#pragma unroll
    for (int i = 1; i < 8; ++i) t = t + red[i][threadIdx.x];
    partial[(int64_t)blockIdx.y * K + col] = t;
  }
}

// acc[k] += the slabs' sums of channel k, added in slab order.
__global__ __launch_bounds__(256) void sumsq_finish_kernel(const double* __restrict__ partial, int64_t slabs,
                                                           int64_t K, double* __restrict__ acc) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= K) return;
  double t = partial[col];
  for (int64_t z = 1; z < slabs; ++z) t = t + partial[z * K + col];
  acc[col] = acc[col] + t;
}

}  // namespace

hipError_t launch_master(const MasterParams& p, hipStream_t s) {
  const int64_t nb = (p.K + 127) / 128;
  const int64_t hpr = nb * 16;  // half groups per row
  const int64_t blocks = (p.N * hpr + 255) / 256;
  if (p.flips || p.risk_hist)
    hipLaunchKernelGGL(master_kernel<true>, dim3((uint32_t)blocks), dim3(256), 0, s, p, (int32_t)hpr);
  else
    hipLaunchKernelGGL(master_kernel<false>, dim3((uint32_t)blocks), dim3(256), 0, s, p, (int32_t)hpr);
  return hipGetLastError();
}

hipError_t launch_master_multi(const MasterParams* ps, int n, hipStream_t s) {
  if (n < 1 || n > kOsciMultiMax) return hipErrorInvalidValue;
  MasterMulti m;
  memset(&m, 0, sizeof(m));
  m.n = n;
  int64_t total = 0;
  bool diag = false;
  for (int i = 0; i < n; ++i) {
    m.p[i] = ps[i];
    const int64_t hpr = (ps[i].K + 127) / 128 * 16;  // half groups per row
    m.hpr[i] = (int32_t)hpr;
    m.begin[i] = (uint32_t)total;
    total += (ps[i].N * hpr + 255) / 256;
    diag = diag || ps[i].flips || ps[i].risk_hist;
  }
  if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  m.begin[n] = (uint32_t)total;
  if (diag)
    hipLaunchKernelGGL(master_multi_kernel<true>, dim3((uint32_t)total), dim3(256), 0, s, m);
  else
    hipLaunchKernelGGL(master_multi_kernel<false>, dim3((uint32_t)total), dim3(256), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_osci(const OsciParams& p, hipStream_t s) {
  const int64_t nb = (p.K + 127) / 128;
  const int64_t hpr = nb * 16;  // half groups per row
  const int64_t blocks = (p.N * hpr + 255) / 256;
  if (p.flips || p.risk_hist)
    hipLaunchKernelGGL(osci_kernel<true>, dim3((uint32_t)blocks), dim3(256), 0, s, p, (int32_t)hpr);
  else
    hipLaunchKernelGGL(osci_kernel<false>, dim3((uint32_t)blocks), dim3(256), 0, s, p, (int32_t)hpr);
  return hipGetLastError();
}

hipError_t launch_osci_multi(const OsciParams* ps, int n, hipStream_t s) {
  if (n < 1 || n > kOsciMultiMax) return hipErrorInvalidValue;
  OsciMulti m;
  memset(&m, 0, sizeof(m));
  m.n = n;
  int64_t total = 0;
  bool diag = false;
  for (int i = 0; i < n; ++i) {
    m.p[i] = ps[i];
    const int64_t hpr = (ps[i].K + 127) / 128 * 16;  // half groups per row
    m.hpr[i] = (int32_t)hpr;
    m.begin[i] = (uint32_t)total;
    total += (ps[i].N * hpr + 255) / 256;
    diag = diag || ps[i].flips || ps[i].risk_hist;
  }
  if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  m.begin[n] = (uint32_t)total;
  if (diag)
    hipLaunchKernelGGL(osci_multi_kernel<true>, dim3((uint32_t)total), dim3(256), 0, s, m);
  else
    hipLaunchKernelGGL(osci_multi_kernel<false>, dim3((uint32_t)total), dim3(256), 0, s, m);
  return hipGetLastError();
}

size_t sumsq_workspace_bytes(int64_t M, int64_t K) {
  return (size_t)((M + kSumsqRows - 1) / kSumsqRows) * (size_t)K * sizeof(double);
}

hipError_t launch_channel_sumsq(const void* X, int64_t M, int64_t K, double* acc, double* partial, hipStream_t s) {
  const int64_t slabs = (M + kSumsqRows - 1) / kSumsqRows;
  const dim3 grid((uint32_t)((K + 255) / 256), (uint32_t)slabs);
  hipLaunchKernelGGL(sumsq_partial_kernel, grid, dim3(256), 0, s, reinterpret_cast<const uint16_t*>(X), M, K, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sumsq_finish_kernel, dim3((uint32_t)((K + 255) / 256)), dim3(256), 0, s, partial, slabs, K, acc);
  return hipGetLastError();
}

}  // namespace tj2
