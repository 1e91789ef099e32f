// Device codecs for the CSA2 path on gfx950: OCP E4M3 ("FN": max 448, no
// infinities) and OCP MX E2M1, written from the format definitions with bit
// manipulation and fixed rounding thresholds.  Rounding is to nearest, ties to
// even, saturating; the sign of the input is always kept.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// ---------------------------------------------------------------- E4M3 encode
// Normal range: round the fp32 mantissa to 3 bits (nearest, ties to even).
// Subnormal range (|x| < 2^-6): the code is rint(|x| * 2^9), exact scaling.
// |x| >= 448 and any rounding above 448 saturate to 0x7E.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {
    mag = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8; 8 is code 0x08 = 2^-6
  } else {
    const uint32_t ua = u & 0x7FFFFFFFu;
    const uint32_t keep = ua >> 20;           // exponent (8b) and top 3 mantissa bits
    const uint32_t rem = ua & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & (keep & 1u));
    const uint32_t r = keep + up;             // a mantissa carry bumps the exponent
    // fp32 exponent bias 127 -> E4M3 bias 7: subtract 120 << 3 from (exp << 3 | m)
    mag = r - (120u << 3);
    if (mag > 0x7Eu) mag = 0x7Eu;
  }
  return sign | mag;
}

// ---------------------------------------------------------------- E4M3 decode
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if (e == 0)
    v = (float)m * 0.001953125f;  // m * 2^-9
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------- E2M1 encode
// Magnitude codes 0..7 = {0, .5, 1, 1.5, 2, 3, 4, 6}; the code is the number of
// decision thresholds passed.  A threshold that is a tie point between an odd
// and an even code is passed only strictly when the lower code is even
// (0.25, 1.25, 2.5, 5.0) and already at equality when the upper one is
// (0.75, 1.75, 3.5).
__device__ __forceinline__ uint32_t e2m1_encode(float q) {
  const uint32_t u = __float_as_uint(q);
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
               (a > 5.0f);
  return ((u >> 28) & 8u) | c;
}

__device__ __forceinline__ float e2m1_decode(uint32_t nib) {
  // 0, .5, 1, 1.5, 2, 3, 4, 6 as (exponent, mantissa) pairs
  const uint32_t m = nib & 7u;
  float v;
  if (m < 2)
    v = 0.5f * (float)m;
  else
    v = __uint_as_float(((126u + (m >> 1)) << 23) | ((m & 1u) << 22));
  return (nib & 8u) ? -v : v;
}

// fp32 -> monotone u32 order key (larger key = larger value); -0 maps like +0.
// Finite values map to keys >= 1, so 0 can mark "no entry".
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

}  // namespace csa2
