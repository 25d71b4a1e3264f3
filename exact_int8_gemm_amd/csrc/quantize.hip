// Per-row int8 activation quantizer (StartLux-Prism README, "Quick start":
// int8 activation ranges; the per-row absmax form is the reading used here).
//
// One workgroup owns one row and spreads it over up to 16 waves, so that a
// few hundred rows already give every SIMD several waves to hide HBM latency
// with.  Each thread loads CPT float4 of the row with 16-byte loads and keeps
// them in registers, the absmax is reduced within each wave (shuffles) and
// across waves (LDS, one barrier; max is exact and order-free), then the
// codes are written with one 4-byte store per float4.  Rows longer than
// 1024 * 4 * kMaxCpt floats take a two-pass variant that reads the row twice.
//
// Arithmetic per row (IEEE fp32, round to nearest even, no flushing):
//   s = amax / 127;  q = clamp(rint(x / s), -127, 127)
// with a NaN scale and zero codes for a row holding a non-finite value, and
// zero codes when s == 0.  x / s is the correctly rounded quotient; the codes
// come from a multiplication by 1/s except next to rounding ties (quant_math.h).
//
// Static form (the README's ranges measured once, ahead of time): one
// caller-given s > 0 for the whole tensor replaces amax / 127; the clamp then
// saturates values beyond the calibrated range (an infinite x or an
// overflowing x / s gives +-127), and only a NaN marks a row (scale NaN,
// zero codes).  The same kernels run both forms; the static one skips the
// absmax and reduces a "no NaN" flag instead.
#include "quant_math.h"
#include "../../include/prism.h"

namespace prism {
namespace {

using namespace quant;

constexpr int kMaxThreads = 1024;
constexpr int kMaxCpt = 16;  // float4 per thread kept in registers: K <= 65536

// Row absmax and finiteness over the whole workgroup; every thread gets the
// same answer.
__device__ inline void row_reduce(float& amax, bool& finite) {
  __shared__ float red_max[kMaxThreads / 64];
  __shared__ int red_fin[kMaxThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  amax = wave_max(amax);
  finite = __all(finite);
  if (lane == 0) {
    red_max[wave] = amax;
    red_fin[wave] = finite ? 1 : 0;
  }
  __syncthreads();
  const int nw = (int)(blockDim.x >> 6);
  amax = red_max[0];
  int fin = red_fin[0];
  for (int i = 1; i < nw; ++i) {
    amax = fmaxf(amax, red_max[i]);
    fin &= red_fin[i];
  }
  finite = fin != 0;
}

// Register-resident variant: the row's K/4 float4 are spread over the
// workgroup, chunk c on thread c % blockDim.x, slot c / blockDim.x < CPT.
// STATIC: `fixed` is the tensor's scale and `finite` below means "no NaN".
template <int CPT, bool STATIC>
__global__ __launch_bounds__(kMaxThreads) void quantize_rows_reg(const float* __restrict__ x,
                                                                  int8_t* __restrict__ q, float* __restrict__ s,
                                                                  int64_t K, float fixed) {
  const int64_t row = blockIdx.x;
  const int T = (int)blockDim.x;
  const float4* xr = reinterpret_cast<const float4*>(x + row * K);
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * K);
  const int64_t nchunk = K / 4;

  float4 v[CPT];
  float amax = 0.0f;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t c = threadIdx.x + (int64_t)T * i;
    if (c < nchunk) {
      v[i] = xr[c];
      if (STATIC) {
        finite = finite && nonan4(v[i]);
      } else {
        amax = fmaxf(amax, absmax4(v[i]));
        finite = finite && finite4(v[i]);
      }
    }
  }
  row_reduce(amax, finite);

  const float sc = STATIC ? (finite ? fixed : __builtin_nanf("")) : row_scale(amax, finite);
  if (threadIdx.x == 0) s[row] = sc;
  const bool zero = !finite || sc == 0.0f;
  const float rc = zero ? 0.0f : fast_recip(sc);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t c = threadIdx.x + (int64_t)T * i;
    if (c < nchunk) qr[c] = zero ? 0u : pack4(v[i], sc, rc);
  }
}

// Long rows: first pass reduces, second pass re-reads and quantizes.
template <bool STATIC>
__global__ __launch_bounds__(kMaxThreads) void quantize_rows_2pass(const float* __restrict__ x,
                                                                    int8_t* __restrict__ q, float* __restrict__ s,
                                                                    int64_t K, float fixed) {
  const int64_t row = blockIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + row * K);
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * K);
  const int64_t nchunk = K / 4;

  float amax = 0.0f;
  bool finite = true;
  for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
    const float4 v = xr[c];
    if (STATIC) {
      finite = finite && nonan4(v);
    } else {
      amax = fmaxf(amax, absmax4(v));
      finite = finite && finite4(v);
    }
  }
  row_reduce(amax, finite);

  const float sc = STATIC ? (finite ? fixed : __builtin_nanf("")) : row_scale(amax, finite);
  if (threadIdx.x == 0) s[row] = sc;
  const bool zero = !finite || sc == 0.0f;
  const float rc = zero ? 0.0f : fast_recip(sc);
  for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) qr[c] = zero ? 0u : pack4(xr[c], sc, rc);
}

template <int CPT, bool STATIC>
void launch_reg(const float* x, int8_t* q, float* s, int64_t M, int64_t K, float fixed, hipStream_t st) {
  const int64_t nchunk = K / 4;
  const int64_t per_cpt = (nchunk + CPT - 1) / CPT;
  const int threads = (int)((per_cpt + 63) / 64 * 64);
  quantize_rows_reg<CPT, STATIC><<<(unsigned)M, threads, 0, st>>>(x, q, s, K, fixed);
}

// float4 per thread: at least 2 (two loads in flight per thread), and rows
// spread over about 640 threads when there are few rows, 256 when there are
// many (measured on MI355X at M x K = 512 x 2560, 512 x 9728, 2048 x 5120
// and 8192 x 5120: 14-23% faster than the fewest float4 per thread).
template <bool STATIC>
int launch_rows(const float* x, int8_t* q, float* s, int64_t M, int64_t K, float fixed, hipStream_t st) {
  const int64_t target = M >= 1024 ? 256 : 640;
  int64_t cpt = (K / 4 + target - 1) / target;
  if (cpt < 2) cpt = 2;
  if (cpt > kMaxCpt) cpt = (K / 4 + kMaxThreads - 1) / kMaxThreads;  // long rows: up to 1024 threads
  if (cpt <= 2) launch_reg<2, STATIC>(x, q, s, M, K, fixed, st);
  else if (cpt <= 3) launch_reg<3, STATIC>(x, q, s, M, K, fixed, st);
  else if (cpt <= 4) launch_reg<4, STATIC>(x, q, s, M, K, fixed, st);
  else if (cpt <= 6) launch_reg<6, STATIC>(x, q, s, M, K, fixed, st);
  else if (cpt <= 8) launch_reg<8, STATIC>(x, q, s, M, K, fixed, st);
  else if (cpt <= 12) launch_reg<12, STATIC>(x, q, s, M, K, fixed, st);
  else if (cpt <= kMaxCpt) launch_reg<kMaxCpt, STATIC>(x, q, s, M, K, fixed, st);
  else quantize_rows_2pass<STATIC><<<(unsigned)M, kMaxThreads, 0, st>>>(x, q, s, K, fixed);
  return launch_status();
}

}  // namespace

int launch_quantize_rows(const float* x, int8_t* q, float* s, int64_t M, int64_t K, hipStream_t st) {
  return launch_rows<false>(x, q, s, M, K, 0.0f, st);
}

int launch_quantize_rows_static(const float* x, int8_t* q, float* s, float scale, int64_t M, int64_t K,
                                hipStream_t st) {
  return launch_rows<true>(x, q, s, M, K, scale, st);
}

}  // namespace prism
