// Device-side building blocks of the TetraJet-v2 NVFP4 path for gfx950 (CDNA4).
//
// Formats (TetraJet-v2 technical summary, section 2.A): NVFP4 = E2M1 elements,
// one E4M3 scale per 16 elements, one FP32 scale per 128-element outer block.
// Every function here reproduces one step of the method bit for bit in fp32
// (compiled with -ffp-contract=off): the tests compare its output with an
// independent CPU implementation.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tj2 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr float kTiny = 0x1p-100f;     // outer blocks with amax below this are empty
constexpr float kNvfp4Div = 2688.0f;   // 6 * 448: outer max -> E2M1 max * E4M3 max
constexpr float kFp8Div = 448.0f;      // outer max -> E4M3 max

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// E4M3FN inner scale: smallest E4M3 value >= r, for 0 < r <= 448.
// Returns the value; *code receives the byte.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_round_up(float r, uint32_t* code) {
  if (r < 0x1p-6f) {                    // subnormal E4M3: quantum 2^-9
    float k = ceilf(r * 512.0f);        // exact scaling, k in 1..8
    *code = (uint32_t)k;                // k = 8 is 2^-6 = code 0x08
    return k * 0x1p-9f;
  }
  uint32_t b = (__float_as_uint(r) + 0xFFFFFu) & 0xFFF00000u;  // ceil to 3 mantissa bits
  *code = (b >> 20) - 960u;             // (exp-127+7)<<3 | m3
  return __uint_as_float(b);
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// E2M1 element rounding (|v| <= 6).  Codes: bit 3 sign, bits 2..0 magnitude
// index into {0, .5, 1, 1.5, 2, 3, 4, 6}.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m1_rtn(float v) {
  uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
  float a = fabsf(v);
  uint32_t idx;
  if (a < 1.0f) {
    idx = (uint32_t)rintf(a * 2.0f);    // 0, 0.5, 1 ; ties to even
  } else {
    uint32_t b = __float_as_uint(a);
    b = b + 0x1FFFFFu + ((b >> 22) & 1u);  // RNE to one mantissa bit
    idx = (b >> 22) - 252u;
  }
  return idx | sign;
}

// Stochastic rounding with a 16-bit draw u: up iff float(u) < (|v|-lo)/(hi-lo)*65536.
__device__ __forceinline__ uint32_t e2m1_sr(float v, uint32_t u) {
  uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
  float a = fabsf(v);
  float lo, scale;
  uint32_t idx;
  if (a < 1.0f) {
    lo = floorf(a * 2.0f) * 0.5f;
    idx = (uint32_t)(lo * 2.0f);
    scale = 131072.0f;                  // 65536 / 0.5
  } else {
    uint32_t b = __float_as_uint(a) & 0xFFC00000u;  // truncate to one mantissa bit
    lo = __uint_as_float(b);
    idx = (b >> 22) - 252u;
    scale = __uint_as_float((271u - (b >> 23)) << 23);  // 65536 / 2^(e-1)
  }
  float t = (a - lo) * scale;           // exact
  uint32_t up = ((float)u < t && idx < 7u) ? 1u : 0u;
  return (idx + up) | sign;
}

// ---------------------------------------------------------------------------
// E4M3FN element rounding (|v| <= 448) for the FP8 outlier channels.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fabsf(v);
  if (a < 0x1p-6f) return sign | (uint32_t)rintf(a * 512.0f);
  uint32_t b = __float_as_uint(a);
  b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
  return sign | ((b >> 20) - 960u);
}

__device__ __forceinline__ uint32_t e4m3_sr(float v, uint32_t u) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fabsf(v);
  uint32_t code;
  float t;
  if (a < 0x1p-6f) {
    float x = a * 512.0f;
    float lo = floorf(x);
    code = (uint32_t)lo;
    t = (x - lo) * 65536.0f;
  } else {
    uint32_t b = __float_as_uint(a) & 0xFFF00000u;
    code = (b >> 20) - 960u;
    t = (a - __uint_as_float(b)) * __uint_as_float((273u - (b >> 23)) << 23);  // 65536 / 2^(e-3)
  }
  uint32_t up = ((float)u < t && code < 0x7Eu) ? 1u : 0u;
  return sign | (code + up);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11).  Draw of input element e: block e>>3,
// counter (lo b, hi b, lo offset, hi offset), key (lo seed, hi seed); word
// (e>>1)&3, half e&1 (0 = low 16 bits).
// ---------------------------------------------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                          uint32_t k0, uint32_t k1) {
#pragma unroll
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
  return {c0, c1, c2, c3};
}

// Eight 16-bit draws of the 8-element block b.
__device__ __forceinline__ void draws8(uint64_t b, uint64_t seed, uint64_t offset, uint32_t u[8]) {
  u32x4 w = philox10((uint32_t)b, (uint32_t)(b >> 32), (uint32_t)offset, (uint32_t)(offset >> 32),
                     (uint32_t)seed, (uint32_t)(seed >> 32));
  u[0] = w.x & 0xFFFFu; u[1] = w.x >> 16;
  u[2] = w.y & 0xFFFFu; u[3] = w.y >> 16;
  u[4] = w.z & 0xFFFFu; u[5] = w.z >> 16;
  u[6] = w.w & 0xFFFFu; u[7] = w.w >> 16;
}

// ---------------------------------------------------------------------------
// 16-wide random Hadamard transform, in registers: negate positions whose bit
// is set in `mask`, butterflies h = 1, 2, 4, 8 pairing (i, i+h) -> (a+b, a-b),
// then * 0.25 (TetraJet-v2 technical summary, section 2.C).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rht16(float v[16], uint32_t mask) {
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((mask >> j) & 1u) << 31));
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
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = v[j] * 0.25f;
}

// ---------------------------------------------------------------------------
// Max over the 8 consecutive lanes of an aligned group (DPP: quad swaps, then
// the half-row mirror, which pairs each lane with one in the other quad).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max8_lanes(float x) {
  int xi = __float_as_int(x);
  int y = __builtin_amdgcn_update_dpp(xi, xi, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x = fmaxf(x, __int_as_float(y));
  xi = __float_as_int(x);
  y = __builtin_amdgcn_update_dpp(xi, xi, 0x4E, 0xF, 0xF, false);       // quad_perm [2,3,0,1]
  x = fmaxf(x, __int_as_float(y));
  xi = __float_as_int(x);
  y = __builtin_amdgcn_update_dpp(xi, xi, 0x141, 0xF, 0xF, false);      // row_half_mirror
  return fmaxf(x, __int_as_float(y));
}

// ---------------------------------------------------------------------------
// Double-block scale computation for one 16-element group whose outer block
// max is a_o and own max is a_j.  Produces the E4M3 code, the FP32 outer scale
// S, and the element multiplier inv = 1 / (s * S) (0 for empty groups).
// ---------------------------------------------------------------------------
struct GroupScale { float S; float inv; uint32_t s_code; };

__device__ __forceinline__ GroupScale nvfp4_group_scale(float a_o, float a_j) {
  GroupScale g;
  if (a_o < kTiny) { g.S = 0.0f; g.inv = 0.0f; g.s_code = 0u; return g; }
  g.S = a_o / kNvfp4Div;
  if (a_j == 0.0f) { g.inv = 0.0f; g.s_code = 0u; return g; }
  float six_s = 6.0f * g.S;
  float r = fminf(a_j / six_s, 448.0f);
  uint32_t code;
  float s = e4m3_round_up(r, &code);
  float d = s * g.S;
  g.inv = 1.0f / d;
  g.s_code = code;
  return g;
}

// Scaled element: clamp(y * inv, -6, 6); an empty group keeps only the sign.
__device__ __forceinline__ float nvfp4_scaled(float y, float inv) {
  if (inv == 0.0f) return __uint_as_float(__float_as_uint(y) & 0x80000000u);
  return fminf(fmaxf(y * inv, -6.0f), 6.0f);
}

__device__ __forceinline__ float fp8_scaled(float y, float inv) {
  if (inv == 0.0f) return __uint_as_float(__float_as_uint(y) & 0x80000000u);
  return fminf(fmaxf(y * inv, -448.0f), 448.0f);
}

}  // namespace tj2
