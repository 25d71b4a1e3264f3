// Element arithmetic of the per-row int8 quantizer, shared by the quantizer
// kernels and the fused single-row GEMM (both must give the same codes).
//   s = amax / 127;  q = clamp(rint(x / s), -127, 127)
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

// Four codes packed little-endian into one dword.
__device__ inline uint32_t pack4(const float4 v, float s) {
  uint32_t b0 = (uint32_t)(code_of(v.x, s) & 0xff);
  uint32_t b1 = (uint32_t)(code_of(v.y, s) & 0xff);
  uint32_t b2 = (uint32_t)(code_of(v.z, s) & 0xff);
  uint32_t b3 = (uint32_t)(code_of(v.w, s) & 0xff);
  return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
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
