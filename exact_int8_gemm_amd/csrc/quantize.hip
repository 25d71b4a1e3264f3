// Per-row int8 activation quantizer (StartLux-Prism README, "Quick start":
// int8 activation ranges; the per-row absmax form is the reading used here).
//
// One 64-lane wave owns one row, four rows per 256-thread workgroup.  The
// row is streamed from HBM once with 16-byte loads and kept in registers
// (CPT float4 per lane), the absmax is reduced across the wave (max is exact
// and order-free), then the codes are written with one 4-byte store per
// float4.  Rows longer than 256*kMaxCpt floats take a two-pass variant that
// reads the row twice.
//
// Arithmetic per row (IEEE fp32, round to nearest even, no flushing):
//   s = amax / 127;  q = clamp(rint(x / s), -127, 127)
// with a NaN scale and zero codes for a row holding a non-finite value, and
// zero codes when s == 0.  The division is the correctly rounded one (the
// library is built with correctly rounded fp32 division).
#include "prism_internal.h"
#include "../../include/prism.h"

namespace prism {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kMaxCpt = 40;  // float4 per lane kept in registers: K <= 10240

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

__device__ inline float absmax4(const float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Register-resident variant: the row's nchunk = K/4 float4 are spread over the
// wave, chunk c on lane c % 64, slot c / 64 < CPT.
template <int CPT>
__global__ __launch_bounds__(64 * kRowsPerBlock) void quantize_rows_reg(const float* __restrict__ x,
                                                                        int8_t* __restrict__ q,
                                                                        float* __restrict__ s, int64_t M,
                                                                        int64_t K) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;  // whole wave leaves together
  const float4* xr = reinterpret_cast<const float4*>(x + row * K);
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * K);
  const int64_t nchunk = K / 4;

  float4 v[CPT];
  float amax = 0.0f;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t c = lane + 64 * i;
    if (c < nchunk) {
      v[i] = xr[c];
      amax = fmaxf(amax, absmax4(v[i]));
      finite = finite && finite4(v[i]);
    }
  }
  amax = wave_max(amax);
  finite = __all(finite);

  const float sc = finite ? amax / 127.0f : __builtin_nanf("");
  if (lane == 0) s[row] = sc;
  const bool zero = !finite || sc == 0.0f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t c = lane + 64 * i;
    if (c < nchunk) qr[c] = zero ? 0u : pack4(v[i], sc);
  }
}

// Long rows: first pass reduces, second pass re-reads and quantizes.
__global__ __launch_bounds__(64 * kRowsPerBlock) void quantize_rows_2pass(const float* __restrict__ x,
                                                                          int8_t* __restrict__ q,
                                                                          float* __restrict__ s, int64_t M,
                                                                          int64_t K) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const float4* xr = reinterpret_cast<const float4*>(x + row * K);
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * K);
  const int64_t nchunk = K / 4;

  float amax = 0.0f;
  bool finite = true;
  for (int64_t c = lane; c < nchunk; c += 64) {
    const float4 v = xr[c];
    amax = fmaxf(amax, absmax4(v));
    finite = finite && finite4(v);
  }
  amax = wave_max(amax);
  finite = __all(finite);

  const float sc = finite ? amax / 127.0f : __builtin_nanf("");
  if (lane == 0) s[row] = sc;
  const bool zero = !finite || sc == 0.0f;
  for (int64_t c = lane; c < nchunk; c += 64) qr[c] = zero ? 0u : pack4(xr[c], sc);
}

template <int CPT>
void launch_reg(const float* x, int8_t* q, float* s, int64_t M, int64_t K, hipStream_t st) {
  const unsigned grid = (unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock);
  quantize_rows_reg<CPT><<<grid, 64 * kRowsPerBlock, 0, st>>>(x, q, s, M, K);
}

}  // namespace

int launch_quantize_rows(const float* x, int8_t* q, float* s, int64_t M, int64_t K, hipStream_t st) {
  const int64_t cpt = (K / 4 + 63) / 64;
  if (cpt <= 1) launch_reg<1>(x, q, s, M, K, st);
  else if (cpt <= 2) launch_reg<2>(x, q, s, M, K, st);
  else if (cpt <= 4) launch_reg<4>(x, q, s, M, K, st);
  else if (cpt <= 8) launch_reg<8>(x, q, s, M, K, st);
  else if (cpt <= 12) launch_reg<12>(x, q, s, M, K, st);
  else if (cpt <= 16) launch_reg<16>(x, q, s, M, K, st);
  else if (cpt <= 24) launch_reg<24>(x, q, s, M, K, st);
  else if (cpt <= 32) launch_reg<32>(x, q, s, M, K, st);
  else if (cpt <= kMaxCpt) launch_reg<kMaxCpt>(x, q, s, M, K, st);
  else {
    const unsigned grid = (unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock);
    quantize_rows_2pass<<<grid, 64 * kRowsPerBlock, 0, st>>>(x, q, s, M, K);
  }
  return launch_status();
}

}  // namespace prism
