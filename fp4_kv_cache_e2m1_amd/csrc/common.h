// Device-side helpers shared by the CSA2 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA2_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace csa2 {

constexpr int kWave = 64;
constexpr int kGroup = 16;  // channels per E4M3 scale

// ---- E4M3 (OCP "FN") -------------------------------------------------------------------------
// Magnitude of an E4M3 code's low 7 bits (0x00..0x7E finite) as fp32, built from its bit
// fields: exponent field 0 is subnormal (m * 2^-9), otherwise (1 + m/8) * 2^(e-7).
CSA2_DEV float e4m3_mag(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9, exact
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Full E4M3 decode of a byte: sign bit 7, and 0x7F / 0xFF are NaN (the format has no infinity).
CSA2_DEV float e4m3_value(uint32_t c) {
  if ((c & 0x7Fu) == 0x7Fu) return __uint_as_float(0x7FC00000u);
  const float v = e4m3_mag(c);
  return (c & 0x80u) ? -v : v;
}

// Nearest E4M3 code to amax / 6 (ties to the even code, saturating at 448), decided by exact
// fp32 comparisons of amax against 6 * value and 3 * (value_lo + value_hi); both products have
// at most 8 significant bits and are exact.
CSA2_DEV uint32_t e4m3_scale_code(float amax) {
  float t = amax * (1.0f / 6.0f);  // estimate; corrected below
  uint32_t c;
  if (!(t < 448.0f)) {
    c = 0x7E;
  } else if (t < 0.015625f) {  // below 2^-6: subnormal codes m * 2^-9
    c = (uint32_t)(t * 512.0f);
  } else {
    uint32_t b = __float_as_uint(t);
    c = ((((b >> 23) & 0xFF) - 120u) << 3) | ((b >> 20) & 7u);
  }
  if (c > 0x7E) c = 0x7E;
  // floor code: largest c with 6 * value(c) <= amax
  while (c > 0 && 6.0f * e4m3_mag(c) > amax) --c;
  while (c < 0x7E && 6.0f * e4m3_mag(c + 1) <= amax) ++c;
  if (c < 0x7E) {
    float mid6 = 3.0f * (e4m3_mag(c) + e4m3_mag(c + 1));
    if (amax > mid6 || (amax == mid6 && ((c + 1) & 1u) == 0)) ++c;
  }
  return c;
}

// ---- E2M1 -------------------------------------------------------------------------------------
// Magnitude code (0..7) of |x| for a scale s > 0: the E2M1 magnitude nearest to |x|/s with ties
// to the even code, via exact compares against s * {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}.
// Thresholds between an odd code and the next even code count ">=" (a tie goes up to the even
// code); the others count ">" (a tie stays on the even code).
// The seven predicates are monotone (the thresholds strictly increase for s >= 2^-9, and every
// product is exact), so the code is the number of them that hold, found by a three-step binary
// search: 1.75 s first, then 0.75 s or 3.5 s, then one of the ">" thresholds.
CSA2_DEV uint32_t e2m1_mag_code(float ax, float s) {
  const bool hi = ax >= 1.75f * s;
  const bool b2 = ax >= (hi ? 3.5f : 0.75f) * s;
  const float t3 = hi ? (b2 ? 5.0f : 2.5f) : (b2 ? 1.25f : 0.25f);
  const bool b3 = ax > t3 * s;
  return (hi ? 4u : 0u) + (b2 ? 2u : 0u) + (b3 ? 1u : 0u);
}

// Twice the E2M1 magnitude of codes 0..7 is {0,1,2,3,4,6,8,12}: bytes of two words, looked up
// with v_perm (4 nibbles per lookup).
constexpr uint32_t kE2M1x2Lo = 0x03020100u;  // codes 0..3 -> 0,1,2,3
constexpr uint32_t kE2M1x2Hi = 0x0C080604u;  // codes 4..7 -> 4,6,8,12

// Eight E2M1 codes (one 32-bit word, channel 2i in the low nibble of byte i) times a scale,
// as eight fp32 values (exact).
CSA2_DEV void e2m1x8_to_f32(uint32_t w, float half_scale, float* out) {
  // magnitude indices of the 8 nibbles, as bytes: even nibbles then odd nibbles
  uint32_t even = w & 0x07070707u;          // channels 0,2,4,6 (low nibbles)
  uint32_t odd = (w >> 4) & 0x07070707u;    // channels 1,3,5,7
  uint32_t me = __builtin_amdgcn_perm(kE2M1x2Hi, kE2M1x2Lo, even);
  uint32_t mo = __builtin_amdgcn_perm(kE2M1x2Hi, kE2M1x2Lo, odd);
  uint32_t se = w & 0x08080808u, so = (w >> 4) & 0x08080808u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float ve = (float)((me >> (8 * i)) & 0xFF) * half_scale;
    float vo = (float)((mo >> (8 * i)) & 0xFF) * half_scale;
    out[2 * i] = (se >> (8 * i)) & 8 ? -ve : ve;
    out[2 * i + 1] = (so >> (8 * i)) & 8 ? -vo : vo;
  }
}

// ---- cross-lane reductions ------------------------------------------------------------------
// Sum over aligned groups of 8 lanes via DPP (quad_perm xor 1, xor 2, then row_half_mirror);
// every lane of the group receives the sum.
CSA2_DEV float sum8(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  return v;
}

CSA2_DEV float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

// Order-preserving 32-bit key of an fp32 score (larger score -> larger key); -0 maps like +0.
// Key 0 is never produced by a finite or infinite score and marks "not a candidate".
CSA2_DEV uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
CSA2_DEV float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

}  // namespace csa2
