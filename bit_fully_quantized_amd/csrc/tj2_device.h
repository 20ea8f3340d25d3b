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

#include <type_traits>
#include <utility>

namespace tj2 {

// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(<N-1>), so that
// register arrays are only ever indexed with constants.
template <class F, int... Ks>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Ks...>) {
  (f(std::integral_constant<int, Ks>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr float kTiny = 0x1p-100f;     // outer blocks with amax below this are empty
constexpr float kNvfp4Div = 2688.0f;   // 6 * 448: outer max -> E2M1 max * E4M3 max
constexpr float kNvfp6Div = 3360.0f;   // 7.5 * 448: outer max -> E2M3 max * E4M3 max
constexpr float kFp8Div = 448.0f;      // outer max -> E4M3 max

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// a * b for 0 <= a, b < 2^32: one 32 x 32 -> 64-bit multiply (a 64 x 64-bit
// product costs three quarter-rate instructions)
__device__ __forceinline__ uint64_t mul32(int64_t a, int64_t b) { return (uint64_t)(uint32_t)a * (uint32_t)b; }

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

// Value of an E4M3FN byte (finite codes).  gfx950's v_cvt_scalef32_pk_f32_fp8
// with scale 1.0 is exact on them: every E4M3 value is an fp32 value.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  typedef float float2_t __attribute__((ext_vector_type(2)));
  const float2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, false);
  return v.x;
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

// Round-to-nearest of 16 scaled values (v = y * inv, unclamped) into 8 bytes of
// E2M1 codes (element 2i in the low nibble of byte i).  gfx950's
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds to nearest-even, saturates at
// +-6 (the clamp) and keeps the sign of zero: the same rule as e2m1_rtn, checked
// exhaustively against it.
__device__ __forceinline__ void e2m1_rtn16(const float y[16], uint32_t out[2]) {
  uint32_t c0 = 0u, c1 = 0u;
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, y[0], y[1], 1.0f, 0);
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, y[2], y[3], 1.0f, 1);
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, y[4], y[5], 1.0f, 2);
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, y[6], y[7], 1.0f, 3);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, y[8], y[9], 1.0f, 0);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, y[10], y[11], 1.0f, 1);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, y[12], y[13], 1.0f, 2);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, y[14], y[15], 1.0f, 3);
  out[0] = c0;
  out[1] = c1;
}

// Stochastic rounding of 16 scaled values with 16-bit draws r[t] held in the
// top half of a 32-bit word (low half zero).  Rule: with t = 65536 * (position of
// |y| inside its grid gap), round up iff u + floor(t) >= 65536.  gfx950's
// v_cvt_scalef32_sr_pk_fp4_f32 rounds up iff the gap fraction plus r / 2^32
// reaches 1, which with r = u << 16 is exactly that rule (checked bit-exactly
// at every threshold against the CPU rule); it also saturates at +-6.  One
// element per instruction (the second slot converts 0.0, code 0), so every
// element gets its own draw.  The instruction leaves bytes 1..3 of its result
// undefined (it does not merge into an old value), so only byte 0 is used:
// pairs are merged with a shift-or, then bytes are gathered with v_perm.  The
// draw doubles as the old value, so no register is cleared for it.
__device__ __forceinline__ uint32_t e2m1_sr1(float y, uint32_t r) {
  typedef float float2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(r, float2_t{y, 0.0f}, r, 1.0f, 0);
}

__device__ __forceinline__ uint32_t e2m1_sr8(const float* y, const uint32_t* r) {
  // byte 0 of each pair word = code(2i) | code(2i+1) << 4; upper bytes are don't-care
  const uint32_t p0 = e2m1_sr1(y[0], r[0]) | (e2m1_sr1(y[1], r[1]) << 4);
  const uint32_t p1 = e2m1_sr1(y[2], r[2]) | (e2m1_sr1(y[3], r[3]) << 4);
  const uint32_t p2 = e2m1_sr1(y[4], r[4]) | (e2m1_sr1(y[5], r[5]) << 4);
  const uint32_t p3 = e2m1_sr1(y[6], r[6]) | (e2m1_sr1(y[7], r[7]) << 4);
  // v_perm_b32(a, b, sel): selector bytes 0-3 pick bytes of b, 4-7 bytes of a
  const uint32_t lo = __builtin_amdgcn_perm(p1, p0, 0x0C0C0400u);  // [p0.b0, p1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(p3, p2, 0x04000C0Cu);  // [0, 0, p2.b0, p3.b0]
  return lo | hi;
}

__device__ __forceinline__ void e2m1_sr16(const float y[16], const uint32_t r[16], uint32_t out[2]) {
  out[0] = e2m1_sr8(y, r);
  out[1] = e2m1_sr8(y + 8, r + 8);
}

// ---------------------------------------------------------------------------
// E4M3FN element rounding (|v| <= 448) for the FP8 outlier channels:
// nearest, ties to even code, sign kept.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fabsf(v);
  if (a < 0x1p-6f) return sign | (uint32_t)rintf(a * 512.0f);
  uint32_t b = __float_as_uint(a);
  b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
  return sign | ((b >> 20) - 960u);
}

// The same rounding for 16 values (|y| <= 448) into 16 bytes with gfx950's
// v_cvt_scalef32_pk_fp8_f32 at scale 1.0, which agrees with e4m3_rne on every
// fp32 value of magnitude <= 448, both signs (checked exhaustively).  Each
// instruction writes one 16-bit half of its destination and keeps the other.
__device__ __forceinline__ void e4m3_rne16(const float y[16], uint32_t out[4]) {
  typedef short short2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    short2_t d = {0, 0};
    d = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(d, y[4 * w + 0], y[4 * w + 1], 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(d, y[4 * w + 2], y[4 * w + 3], 1.0f, true);
    out[w] = __builtin_bit_cast(uint32_t, d);
  }
}

// Same rule on the E4M3 grid with v_cvt_scalef32_sr_fp8_f32 (one element per
// instruction, byte `sel` of the destination).  The instruction does not
// saturate, so inputs are clamped to +-448 by the caller.
__device__ __forceinline__ void e4m3_sr16(const float y[16], const uint32_t r[16], uint32_t out[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t d = 0u;
    d = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d, y[4 * w + 0], r[4 * w + 0], 1.0f, 0);
    d = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d, y[4 * w + 1], r[4 * w + 1], 1.0f, 1);
    d = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d, y[4 * w + 2], r[4 * w + 2], 1.0f, 2);
    d = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d, y[4 * w + 3], r[4 * w + 3], 1.0f, 3);
    out[w] = d;
  }
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
    // three-input xor in one instruction (truth table 0x96)
    uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// Eight 16-bit draws of the 8-element block b, each placed in the top half of
// a 32-bit word (the form the stochastic conversions take).
__device__ __forceinline__ void draws8(uint64_t b, uint64_t seed, uint64_t offset, uint32_t r[8]) {
  u32x4 w = philox10((uint32_t)b, (uint32_t)(b >> 32), (uint32_t)offset, (uint32_t)(offset >> 32),
                     (uint32_t)seed, (uint32_t)(seed >> 32));
  r[0] = w.x << 16; r[1] = w.x & 0xFFFF0000u;
  r[2] = w.y << 16; r[3] = w.y & 0xFFFF0000u;
  r[4] = w.z << 16; r[5] = w.z & 0xFFFF0000u;
  r[6] = w.w << 16; r[7] = w.w & 0xFFFF0000u;
}

// The random Hadamard transform's sign on position j (bit 31 when bit j of
// `mask` is set).
__device__ __forceinline__ uint32_t rht_sign(uint32_t mask, int j) { return ((mask >> j) & 1u) << 31; }

// Butterflies h = 1, 2, 4, 8 pairing (i, i+h) -> (a+b, a-b), then * 0.25: the
// transform after its signs.
__device__ __forceinline__ void hadamard16(float v[16]) {
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
// 16-wide random Hadamard transform, in registers: negate positions whose bit
// is set in `mask`, butterflies h = 1, 2, 4, 8 pairing (i, i+h) -> (a+b, a-b),
// then * 0.25 (TetraJet-v2 technical summary, section 2.C).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rht16(float v[16], uint32_t mask) {
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = __uint_as_float(__float_as_uint(v[j]) ^ rht_sign(mask, j));
  hadamard16(v);
}

// ---------------------------------------------------------------------------
// Max over the 8 consecutive lanes of an aligned group (DPP: quad swaps, then
// the half-row mirror, which pairs each lane with one in the other quad).  The
// inputs are amaxes (>= 0, never NaN), whose fp32 bit patterns order as
// unsigned integers, so each step is one integer max with a DPP operand.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max8_lanes(float x) {
  uint32_t xi = __float_as_uint(x);
  xi = max(xi, (uint32_t)__builtin_amdgcn_mov_dpp((int)xi, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  xi = max(xi, (uint32_t)__builtin_amdgcn_mov_dpp((int)xi, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  xi = max(xi, (uint32_t)__builtin_amdgcn_mov_dpp((int)xi, 0x141, 0xF, 0xF, false));  // row_half_mirror
  return __uint_as_float(xi);
}

// ---------------------------------------------------------------------------
// Double-block scale computation for one 16-element group whose outer block
// max is a_o and own max is a_j.  Produces the E4M3 code, the FP32 outer scale
// S, and the element multiplier inv = 1 / (s * S) (0 for empty groups).
// ---------------------------------------------------------------------------
struct GroupScale { float S; float inv; uint32_t s_code; };

// The element grid's largest value EMAX and the outer divisor EMAX * 448: E2M1 (6, 2688) or E2M3 (7.5, 3360).
template <int FP6>
__device__ __forceinline__ GroupScale double_block_scale(float a_o, float a_j) {
  constexpr float kDiv = FP6 ? kNvfp6Div : kNvfp4Div;
  constexpr float kEmax = FP6 ? 7.5f : 6.0f;
  GroupScale g;
  if (a_o < kTiny) { g.S = 0.0f; g.inv = 0.0f; g.s_code = 0u; return g; }
  g.S = a_o / kDiv;
  if (a_j == 0.0f) { g.inv = 0.0f; g.s_code = 0u; return g; }
  float six_s = kEmax * g.S;
  float r = fminf(a_j / six_s, 448.0f);
  uint32_t code;
  float s = e4m3_round_up(r, &code);
  float d = s * g.S;
  // r below the fp32 range (a group under 2^-149 of its block's scale) gives
  // s = 0: the group then encodes signed zeros, as its scale decodes it
  g.inv = d > 0.0f ? 1.0f / d : 0.0f;
  g.s_code = code;
  return g;
}

__device__ __forceinline__ GroupScale nvfp4_group_scale(float a_o, float a_j) { return double_block_scale<0>(a_o, a_j); }
__device__ __forceinline__ GroupScale nvfp6_group_scale(float a_o, float a_j) { return double_block_scale<1>(a_o, a_j); }

// ---------------------------------------------------------------------------
// E2M3 element rounding (|v| <= 7.5), the FP6 elements of the FP6 x FP4
// variant, returned as the E4M3FN byte of the E2M3 value (every E2M3 value
// is an E4M3 value: 0 and k/8 below 1, three mantissa bits from 1 to 7.5).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_byte_of(float r, uint32_t sign) {
  // r is 0 or an E4M3 normal value (>= 2^-3 here)
  return r == 0.0f ? sign : sign | ((__float_as_uint(r) >> 20) - 960u);
}

// nearest, ties to even mantissa, sign kept
__device__ __forceinline__ uint32_t e2m3_rtn_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  float r;
  if (a < 1.0f) {
    r = rintf(a * 8.0f) * 0.125f;  // grid k/8, ties to even k
  } else {
    uint32_t b = __float_as_uint(a);
    b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;  // RNE to 3 mantissa bits
    r = __uint_as_float(b);
  }
  return e4m3_byte_of(r, sign);
}

// stochastic: with lo <= |v| < hi the neighbouring grid values and
// t = 65536 (|v| - lo) / (hi - lo) (exact), round up iff u + floor(t) >= 65536,
// u the 16-bit draw in the top half of rnd
__device__ __forceinline__ uint32_t e2m3_sr_e4m3(float v, uint32_t rnd) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  float lo, gap;
  if (a < 1.0f) {
    lo = floorf(a * 8.0f) * 0.125f;
    gap = 0.125f;
  } else {
    const uint32_t b = __float_as_uint(a) & 0xFFF00000u;  // truncate to 3 mantissa bits
    lo = __uint_as_float(b);
    gap = __uint_as_float((b & 0x7F800000u) - (3u << 23));  // 2^(e - 3)
  }
  const float t = ((a - lo) / gap) * 65536.0f;  // exact
  const bool up = lo < 7.5f && (rnd >> 16) + (uint32_t)t >= 65536u;
  return e4m3_byte_of(up ? lo + gap : lo, sign);
}

// Scaled element: clamp(y * inv, -6, 6).  An empty group has inv = 0, and
// y * 0 is a zero with the sign of y, so it encodes the sign only.
__device__ __forceinline__ float nvfp4_scaled(float y, float inv) {
  return fminf(fmaxf(y * inv, -6.0f), 6.0f);
}

__device__ __forceinline__ float fp8_scaled(float y, float inv) {
  return fminf(fmaxf(y * inv, -448.0f), 448.0f);
}

}  // namespace tj2
