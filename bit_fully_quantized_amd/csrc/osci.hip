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

// Amaxes of this lane's half (8 elements) of a 16-element group: the group's
// (the lane pair) and the 128-element outer block's (16 lanes).  Called in
// uniform control flow (DPP reads the neighbouring lanes).
__device__ __forceinline__ void half_amax(const float w[8], bool valid, float* a_j, float* a_o) {
  float a_h = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) a_h = fmaxf(a_h, fabsf(w[t]));
  if (!valid) a_h = 0.0f;
  uint32_t ai = __float_as_uint(a_h);
  ai = max(ai, (uint32_t)__builtin_amdgcn_mov_dpp((int)ai, 0xB1, 0xF, 0xF, false));  // the group's other half
  *a_j = __uint_as_float(ai);
  *a_o = max16_lanes(*a_j);
}

// Forward NVFP4 quantization of this lane's 8 elements given the amaxes:
// the lane's 8 codes (one word), the group's E4M3 code and S, and the
// dequantized values Q(w).
__device__ __forceinline__ void nvfp4_encode8(const float w[8], bool valid, float a_j, float a_o, uint32_t* code,
                                              uint32_t* s_code, float* S, float q[8]) {
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

// Forward FP8 quantization (OutControl channels, technical summary section
// 2.C: E4M3, one FP32 scale a_o / 448 per 128 elements, round to nearest
// even) of this lane's 8 elements: two words of codes (element t in byte t)
// and the dequantized values e * S8.
__device__ __forceinline__ void fp8_encode8(const float w[8], bool valid, float a_o, uint32_t code[2], float* S,
                                            float q[8]) {
  typedef short short2_t __attribute__((ext_vector_type(2)));
  typedef float float2_t __attribute__((ext_vector_type(2)));
  float S8 = 0.0f, inv = 0.0f;
  if (a_o >= kTiny) {
    S8 = a_o / kFp8Div;
    inv = 1.0f / S8;
  }
  float y[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) y[t] = fp8_scaled(valid ? w[t] : 0.0f, inv);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    short2_t d = {0, 0};
    d = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(d, y[4 * h + 0], y[4 * h + 1], 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(d, y[4 * h + 2], y[4 * h + 3], 1.0f, true);
    code[h] = __builtin_bit_cast(uint32_t, d);
    const float2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code[h], 1.0f, false);  // exact E4M3 values
    const float2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code[h], 1.0f, true);
    q[4 * h + 0] = lo.x * S8;
    q[4 * h + 1] = lo.y * S8;
    q[4 * h + 2] = hi.x * S8;
    q[4 * h + 3] = hi.y * S8;
  }
  *S = S8;
}

// The forward quantization of this lane's 8 elements in its segment: NVFP4
// (fp8 == false: codes[0], s_code) or FP8 (codes[0..1]).  Amaxes in uniform
// control flow, then the per-lane encode.
__device__ __forceinline__ void fwd_quant8(const float w[8], bool valid, bool fp8, uint32_t codes[2],
                                           uint32_t* s_code, float* S, float q[8]) {
  float a_j, a_o;
  half_amax(w, valid, &a_j, &a_o);
  if (fp8) {
    fp8_encode8(w, valid, a_o, codes, S, q);
    *s_code = 0u;
  } else {
    nvfp4_encode8(w, valid, a_j, a_o, &codes[0], s_code, S, q);
    codes[1] = 0u;
  }
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

// Bin changes between the 8 E4M3 codes of two words pairs; +0 and -0 are one bin.
__device__ __forceinline__ uint32_t code_flips_fp8(const uint32_t c[2], const uint32_t cp[2]) {
  uint32_t n = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t a = (c[h] >> (8 * t)) & 0xFFu, b = (cp[h] >> (8 * t)) & 0xFFu;
      n += (a != b && ((a | b) & 0x7Fu) != 0u) ? 1u : 0u;
    }
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

// Element access of one lane: 8 consecutive elements of a row.  With an
// outlier plan the lane covers 8 consecutive positions of the row's compacted
// channel order (the rest channels, then the outlier channels): the masters W
// and the gradient, which are in channel order, are gathered through the
// plan's index lists; the pass's own state arrays (W_prev, Q_prev, dQ, dM and
// the moments m, v) are kept in the compacted order, so their accesses stay
// contiguous.
template <bool PLAN>
struct Lane8 {
  int64_t idx[8];  // channel-order positions (W, grad)
  int64_t cpos;    // first compacted position (state arrays)
  __device__ __forceinline__ void init(const OsciProblem& q, uint32_t row, uint32_t jl, bool fp8) {
    const int64_t base = (int64_t)row * q.K;
    if (PLAN) {
      const int4* ip = reinterpret_cast<const int4*>((fp8 ? q.outl : q.rest) + jl * 8u);
      const int4 c0 = ip[0], c1 = ip[1];
      idx[0] = base + c0.x; idx[1] = base + c0.y; idx[2] = base + c0.z; idx[3] = base + c0.w;
      idx[4] = base + c1.x; idx[5] = base + c1.y; idx[6] = base + c1.z; idx[7] = base + c1.w;
      cpos = base + (fp8 ? q.K1 : 0) + (int64_t)jl * 8;
    } else {
      cpos = base + (int64_t)jl * 8;
#pragma unroll
      for (int t = 0; t < 8; ++t) idx[t] = cpos + t;
    }
  }
  // W and grad (channel order)
  __device__ __forceinline__ void load_ch(const float* a, float v[8]) const {
    if (PLAN) {
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = a[idx[t]];
    } else {
      load8f(a + cpos, v);
    }
  }
  __device__ __forceinline__ void store_ch(float* a, const float v[8]) const {
    if (PLAN) {
#pragma unroll
      for (int t = 0; t < 8; ++t) a[idx[t]] = v[t];
    } else {
      store8f(a + cpos, v);
    }
  }
  // state arrays (compacted order under a plan): contiguous, 16-byte aligned (K1 and K are multiples of 16)
  __device__ __forceinline__ void load(const float* a, float v[8]) const { load8f(a + cpos, v); }
  __device__ __forceinline__ void store(float* a, const float v[8]) const { store8f(a + cpos, v); }
};

// Codes of the final W: NVFP4 (the rest channels, or all of them without a plan)
// or FP8 (the outlier channels), padding included.
__device__ __forceinline__ void store_codes(const OsciProblem& q, uint32_t row, uint32_t jl, bool fp8,
                                            const uint32_t codes[2], uint32_t s_code, float S) {
  if (fp8) {
    const QOut& o = q.w8;
    if (!o.codes) return;
    *reinterpret_cast<uint2*>(o.codes + (int64_t)row * o.ld_codes + jl * 8u) = make_uint2(codes[0], codes[1]);
    if ((jl & 15u) == 0u) o.s128[(int64_t)row * o.ld_s128 + (jl >> 4)] = S;
  } else {
    const QOut& o = q.wq;
    if (!o.codes) return;
    *reinterpret_cast<uint32_t*>(o.codes + (int64_t)row * o.ld_codes + jl * 4u) = codes[0];
    if ((jl & 1u) == 0u) o.s16[(int64_t)row * o.ld_s16 + (jl >> 1)] = (uint8_t)s_code;
    if ((jl & 15u) == 0u) o.s128[(int64_t)row * o.ld_s128 + (jl >> 4)] = S;
  }
}

// One lane per half group; the 16 lanes of a 128-element outer block are
// consecutive, and an outer block lies in one segment (rest or outliers: each
// segment is padded to whole outer blocks).  All loads of the lane are issued
// before the quantization work.  Lanes past the last row stay (no early exit:
// the DPP reductions and the diagnostics' barriers need every lane) but touch
// no memory.
//
// MASTER == false: OsciReset (section 2.B) of the masters as given.
// MASTER == true:  AdamW on the masters first (fp32, one rounded operation at a
//                  time; the pages use fp32 masters and apply OsciReset after
//                  the update without naming the optimizer), then OsciReset of
//                  the new masters with the pre-update master as W_prev.
template <bool MASTER, bool DIAG, bool PLAN>
__device__ __forceinline__ void osci_body(const OsciShared& c, const OsciProblem& q, uint32_t g, DiagSmem& dsm) {
  const uint32_t row = g / (uint32_t)q.hpr;
  const bool live = row < (uint32_t)q.N;  // whole outer blocks are live or not
  const uint32_t jh = g - row * (uint32_t)q.hpr;
  const bool fp8 = PLAN && jh >= (uint32_t)q.hpr1;         // uniform over an outer block
  const uint32_t jl = fp8 ? jh - (uint32_t)q.hpr1 : jh;    // half group within the segment
  const int32_t len = fp8 ? q.no : q.K1;
  const bool valid = live && (int32_t)(jl >> 1) * 16 < len;
  const bool init = !MASTER && c.mode == TJ2_OSCI_INIT;
  const bool window_end = c.mode == TJ2_OSCI_WINDOW_END;

  Lane8<PLAN> L;
  float w[8], wp[8], qp[8], dq[8], dm[8], m[8], v[8], gr[8];
  if (valid) {
    L.init(q, row, jl, fp8);
    L.load_ch(q.W, w);
    if (MASTER) {
      L.load(q.m, m);
      L.load(q.v, v);
      L.load_ch(q.grad, gr);
    }
    if (!init) {
      if (!MASTER) L.load(q.W_prev, wp);
      L.load(q.Q_prev, qp);
      L.load(q.dQ, dq);
      L.load(q.dM, dm);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) w[t] = 0.0f;
  }
  if (MASTER) {
    // AdamW: wp is the pre-update master, w the new one
    const float omb1 = 1.0f - c.beta1, omb2 = 1.0f - c.beta2;
    const float decay = 1.0f - c.lr * c.weight_decay;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float m1 = c.beta1 * m[t] + omb1 * gr[t];
      const float v1 = c.beta2 * v[t] + omb2 * (gr[t] * gr[t]);
      const float u = (m1 / c.bc1) / (sqrtf(v1 / c.bc2) + c.eps);
      wp[t] = w[t];
      w[t] = valid ? w[t] * decay - c.lr * u : 0.0f;
      m[t] = m1;
      v[t] = v1;
    }
  }
  uint32_t codes[2], s_code;
  float S, qv[8];
  fwd_quant8(w, valid, fp8, codes, &s_code, &S, qv);
  uint32_t codes_prev[2] = {0u, 0u};  // diagnostics: the previous master's codes (a flip is a change of bin)
  if (DIAG && !init) {
    float x[8], qx[8], Sx;
    uint32_t sx;
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = valid ? wp[t] : 0.0f;
    fwd_quant8(x, valid, fp8, codes_prev, &sx, &Sx, qx);
  }

  uint32_t n_reset = 0, n_flip = 0;
  uint32_t bins[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const bool want_bins = DIAG && c.risk_hist && window_end;
  if (valid) {
    if (init) {
      float z[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) z[t] = 0.0f;
      L.store(q.W_prev, w);
      L.store(q.Q_prev, qv);
      L.store(q.dQ, z);
      L.store(q.dM, z);
    } else {
      if (DIAG) n_flip = fp8 ? code_flips_fp8(codes, codes_prev) : code_flips(codes[0], codes_prev[0]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        dq[t] = dq[t] + fabsf(qv[t] - qp[t]);
        dm[t] = dm[t] + fabsf(w[t] - wp[t]);
        wp[t] = w[t];
      }
      bool wrote_w = MASTER;  // the master pass always writes the new masters
      if (window_end) {
        if (want_bins) {
#pragma unroll
          for (int t = 0; t < 8; ++t) bins[t] = risk_bin(dq[t], dm[t]);
        }
        if (c.reset_enabled) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            if (dq[t] > c.tau * dm[t]) {
              w[t] = qv[t];
              wp[t] = qv[t];
              ++n_reset;
            }
          }
          wrote_w = wrote_w || n_reset != 0;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) { dq[t] = 0.0f; dm[t] = 0.0f; }
      }
      if (wrote_w) L.store_ch(q.W, w);
      if (MASTER) {
        L.store(q.m, m);
        L.store(q.v, v);
      } else {
        L.store(q.W_prev, wp);
      }
      L.store(q.Q_prev, qv);
      L.store(q.dQ, dq);
      L.store(q.dM, dm);
    }
  }
  const bool any_reset = max16_lanes(n_reset ? 1.0f : 0.0f) > 0.0f;  // uniform over the outer block
  if (any_reset) fwd_quant8(w, valid, fp8, codes, &s_code, &S, qv);  // scales may change after a reset
  if (live) store_codes(q, row, jl, fp8, codes, s_code, S);
  if (c.reset_count && n_reset) atomicAdd(c.reset_count, (unsigned long long)n_reset);
  if constexpr (DIAG) add_diag(dsm, c.flips, want_bins ? c.risk_hist : nullptr, n_flip, want_bins && valid, bins);
}

// Up to kOsciMultiMax weight matrices per launch (a model's matrices after one
// optimizer step), so that small matrices do not each pay a launch:
// workgroups [begin[i], begin[i+1]) take problem i.  Problems with and
// without an outlier plan may share a launch (the branch is uniform per
// workgroup).
template <bool MASTER, bool DIAG>
__global__ __launch_bounds__(256) void osci_multi_kernel(OsciLaunch L) {
  __shared__ DiagSmem dsm;
  int i = 0;
  while (i + 1 < L.n && blockIdx.x >= L.begin[i + 1]) ++i;  // uniform per workgroup
  const uint32_t g = (blockIdx.x - L.begin[i]) * 256u + threadIdx.x;
  if (L.p[i].rest) osci_body<MASTER, DIAG, true>(L.c, L.p[i], g, dsm);
  else osci_body<MASTER, DIAG, false>(L.c, L.p[i], g, dsm);
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

hipError_t launch_osci_multi(const OsciShared& c, const OsciProblem* ps, int n, bool master, hipStream_t s) {
  if (n < 1 || n > kOsciMultiMax) return hipErrorInvalidValue;
  OsciLaunch L;
  memset(&L, 0, sizeof(L));
  L.c = c;
  L.n = n;
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    L.p[i] = ps[i];
    L.begin[i] = (uint32_t)total;
    total += ((int64_t)ps[i].N * ps[i].hpr + 255) / 256;
  }
  if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  L.begin[n] = (uint32_t)total;
  const bool diag = c.flips || c.risk_hist;
  const dim3 grid((uint32_t)total);
  if (master) {
    if (diag) hipLaunchKernelGGL((osci_multi_kernel<true, true>), grid, dim3(256), 0, s, L);
    else hipLaunchKernelGGL((osci_multi_kernel<true, false>), grid, dim3(256), 0, s, L);
  } else {
    if (diag) hipLaunchKernelGGL((osci_multi_kernel<false, true>), grid, dim3(256), 0, s, L);
    else hipLaunchKernelGGL((osci_multi_kernel<false, false>), grid, dim3(256), 0, s, L);
  }
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
