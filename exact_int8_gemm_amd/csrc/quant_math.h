// Element arithmetic of the per-row int8 quantizer, shared by the quantizer
// kernels and the fused single-row GEMM (both must give the same codes).
//   s = amax / 127;  q = clamp(rint(x / s), -127, 127)
// where x / s is the correctly rounded quotient (code_of); code_fast gets the
// same code from a multiplication by 1/s in all but the rare elements next to
// a rounding tie.
// IEEE fp32, round to nearest even, no flushing; the division is the
// correctly rounded one (the library is built with correctly rounded fp32
// division).
#pragma once

#include "prism_internal.h"

namespace prism {
namespace quant {

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ inline int code_of(float x, float s) {
  float r = rintf(x / s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

// The same code from r = 1/s (correctly rounded) without the division, for
// a scale s in [2^-126, 2^126] (r is then a normal float).  t = x * r differs
// from x / s by at most 2^-16 when |x / s| <= 128, and the correctly rounded
// quotient q = fl(x / s) differs from x / s by at most 2^-17, so |t - q| <
// 2^-15.  If t is farther than that from every half-integer, t and q lie
// strictly on the same side of each one and rint(t) == rint(q); the distance
// |t - rint(t)| is computed exactly (t and rint(t) are multiples of t's ulp).
// Otherwise (a rounding tie may be near) the quotient is computed exactly.
// For |x / s| > 128 both t and q exceed 127.5 in magnitude and clamp to the
// same code.  An infinite x (static scales only) gives a NaN distance and
// takes the exact path.
__device__ inline int code_fast(float x, float s, float r) {
  const float t = x * r;
  const float n = rintf(t);
  if (!(fabsf(t - n) < 0.5f - 0x1p-15f)) return code_of(x, s);
  return (int)fminf(fmaxf(n, -127.0f), 127.0f);
}

// 1/s for code_fast, or 0 when s is outside [2^-126, 2^126] (then every
// code takes the division).
__device__ inline float fast_recip(float s) { return (s >= 0x1p-126f && s <= 0x1p126f) ? 1.0f / s : 0.0f; }

// Four codes packed little-endian into one dword; r = fast_recip(s).  The
// four codes come from code_fast's multiplication unless one of them lies
// next to a rounding tie (or r == 0): then all four take the division, in a
// branch that is rarely entered (as one branch for the four, rather than one
// per element, it stays a branch instead of being computed for every
// element and selected).
__device__ inline uint32_t pack4(const float4 v, float s, float r) {
  const float xs[4] = {v.x, v.y, v.z, v.w};
  int c[4];
  bool exact = r == 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float t = xs[e] * r;
    const float n = rintf(t);
    exact = exact || !(fabsf(t - n) < 0.5f - 0x1p-15f);
    c[e] = (int)fminf(fmaxf(n, -127.0f), 127.0f);
  }
  if (__builtin_expect(exact, 0)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = code_of(xs[e], s);
  }
  return (uint32_t)(c[0] & 0xff) | ((uint32_t)(c[1] & 0xff) << 8) | ((uint32_t)(c[2] & 0xff) << 16) |
         ((uint32_t)(c[3] & 0xff) << 24);
}

__device__ inline bool finite4(const float4 v) {
  return isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w);
}

__device__ inline bool nonan4(const float4 v) {
  return !isnan(v.x) && !isnan(v.y) && !isnan(v.z) && !isnan(v.w);
}

__device__ inline float absmax4(const float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// The row scale from the row's absmax and finiteness: NaN for a row with a
// non-finite value (its codes are then 0, as they are when the scale is 0).
__device__ inline float row_scale(float amax, bool finite) {
  return finite ? amax / 127.0f : __builtin_nanf("");
}

}  // namespace quant
}  // namespace prism
