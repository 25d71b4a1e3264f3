// Small-M GEMM (M <= 64): W8A8 and W4A8 with per-channel scales.
//
// Exact int32 sums (StartLux-Prism README, "Why StartLux-Prism" and "How it
// works") make a split of K free: integer addition is associative, so any
// grouping of the k-range gives the same accumulator.  At small M the weights
// dominate the bytes, so this kernel is built to stream them from HBM:
//
//  * one workgroup owns 16 output columns and all M rows; its WAVES waves
//    split K into contiguous ranges and reduce their int32 partials in LDS;
//  * weights go from HBM straight into MFMA operand registers with 16-byte
//    loads (no LDS staging: each weight byte is used by one wave only), four
//    128-k units at a time so that many loads are in flight per wave;
//  * v_mfma_i32_16x16x64_i8: lane l holds column (l % 16) of the weights and
//    row (l % 16) of the activations, k-group l / 16.  Both operands use the
//    same lane -> k assignment, so the integer sum is the plain dot product
//    whatever that assignment is.  Lane group g covers k = unit*128 + 32g +
//    [0, 16) in the first MFMA of a unit and + [16, 32) in the second;
//  * 4-bit weights are unpacked in registers: each nibble is moved to the top
//    half of a byte, which as int8 equals 16 * w, so the MFMA sums 16 * acc
//    exactly (|16 * acc| < 2^31 for K <= 131040) and an arithmetic shift by 4
//    recovers acc;
//  * epilogue per element, in a fixed order: y = ((float)acc * s_a[m]) * s_w[n].
#include "prism_internal.h"
#include "../../include/prism.h"

namespace prism {
namespace {

constexpr int kUnitK = 128;
constexpr int kUnroll = 4;

__device__ inline v4i load16(const int8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// 16 packed bytes = 32 nibbles, k ascending, low nibble first ->
// two 16-byte fragments of int8 (16 * w) in k order.
__device__ inline void unpack_w4(const v4i p, v4i& lo, v4i& hi) {
  int o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = (uint32_t)p[j];
    const uint32_t L = (u << 4) & 0xF0F0F0F0u;  // even k: low nibbles, moved up
    const uint32_t H = u & 0xF0F0F0F0u;         // odd k: high nibbles, in place
    // byte order of the output: L0 H0 L1 H1 | L2 H2 L3 H3
    o[2 * j] = (int)__builtin_amdgcn_perm(H, L, 0x05010400u);
    o[2 * j + 1] = (int)__builtin_amdgcn_perm(H, L, 0x07030602u);
  }
  lo = v4i{o[0], o[1], o[2], o[3]};
  hi = v4i{o[4], o[5], o[6], o[7]};
}

template <int MB, bool W4, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemm_small_kernel(const int8_t* __restrict__ q,
                                                                const float* __restrict__ s_a,
                                                                const int8_t* __restrict__ w,
                                                                const float* __restrict__ s_w,
                                                                float* __restrict__ y,
                                                                int32_t* __restrict__ acc_out, int M, int N,
                                                                int K) {
  __shared__ int red[WAVES][MB * 4][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int n = n0 + col;
  const bool nvalid = n < N;

  const int nunits = (K + kUnitK - 1) / kUnitK;
  const int ub = (int)((int64_t)wave * nunits / WAVES);
  const int ue = (int)((int64_t)(wave + 1) * nunits / WAVES);

  v4i acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = v4i{0, 0, 0, 0};

  const int8_t* wrow = w + (W4 ? (size_t)n * (size_t)(K / 2) : (size_t)n * (size_t)K);

  for (int u0 = ub; u0 < ue; u0 += kUnroll) {
    v4i b0[kUnroll], b1[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int kk = (u0 + j) * kUnitK + g * 32;
      b0[j] = v4i{0, 0, 0, 0};
      b1[j] = v4i{0, 0, 0, 0};
      if (u0 + j < ue && nvalid) {
        if (W4) {
          if (kk < K) unpack_w4(load16(wrow + kk / 2), b0[j], b1[j]);
        } else {
          if (kk < K) b0[j] = load16(wrow + kk);
          if (kk + 16 < K) b1[j] = load16(wrow + kk + 16);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      if (u0 + j >= ue) break;  // uniform over the wave
      const int kk = (u0 + j) * kUnitK + g * 32;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = mb * 16 + col;
        v4i a0 = v4i{0, 0, 0, 0}, a1 = v4i{0, 0, 0, 0};
        if (m < M) {
          const int8_t* qr = q + (size_t)m * (size_t)K;
          if (kk < K) a0 = load16(qr + kk);
          if (kk + 16 < K) a1 = load16(qr + kk + 16);
        }
        acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0[j], acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1[j], acc[mb], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][mb * 4 + i][lane] = acc[mb][i];
  __syncthreads();

  // Output layout of the 16x16 MFMA: lane l, register i -> row 4 * (l / 16) + i,
  // column l % 16.
  for (int e = threadIdx.x; e < MB * 4 * 64; e += 64 * WAVES) {
    const int mbi = e >> 6;
    const int l = e & 63;
    int s = 0;
#pragma unroll
    for (int wv = 0; wv < WAVES; ++wv) s += red[wv][mbi][l];
    if (W4) s >>= 4;  // exact: the sum is a multiple of 16
    const int m = (mbi >> 2) * 16 + (l >> 4) * 4 + (mbi & 3);
    const int nn = n0 + (l & 15);
    if (m < M && nn < N) {
      const size_t o = (size_t)m * (size_t)N + (size_t)nn;
      if (acc_out) acc_out[o] = s;
      const float t = (float)s * s_a[m];
      y[o] = t * s_w[nn];
    }
  }
}

template <int MB, bool W4, int WAVES>
void launch_small(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y,
                  int32_t* acc, int M, int N, int K, hipStream_t st) {
  const unsigned grid = (unsigned)((N + 15) / 16);
  gemm_small_kernel<MB, W4, WAVES><<<grid, 64 * WAVES, 0, st>>>(q, s_a, w, s_w, y, acc, M, N, K);
}

template <int MB, bool W4>
void pick_waves(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc,
                int M, int N, int K, hipStream_t st) {
  // Aim for about 16 waves per CU over the 256 CUs, without giving a wave
  // less than two 128-k units.
  const int64_t nwg = (N + 15) / 16;
  const int64_t nunits = (K + kUnitK - 1) / kUnitK;
  int waves = 4;
  if (nwg * 8 <= 4096 && nunits >= 16) waves = 8;
  if (nwg * 16 <= 4096 && nunits >= 32) waves = 16;
  if (waves == 16) launch_small<MB, W4, 16>(q, s_a, w, s_w, y, acc, M, N, K, st);
  else if (waves == 8) launch_small<MB, W4, 8>(q, s_a, w, s_w, y, acc, M, N, K, st);
  else launch_small<MB, W4, 4>(q, s_a, w, s_w, y, acc, M, N, K, st);
}

template <bool W4>
void pick_mb(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc,
             int M, int N, int K, hipStream_t st) {
  if (M <= 16) pick_waves<1, W4>(q, s_a, w, s_w, y, acc, M, N, K, st);
  else if (M <= 32) pick_waves<2, W4>(q, s_a, w, s_w, y, acc, M, N, K, st);
  else pick_waves<4, W4>(q, s_a, w, s_w, y, acc, M, N, K, st);
}

}  // namespace

int launch_gemm_small(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                      float* y, int32_t* acc, int M, int N, int K, hipStream_t st) {
  const int8_t* wb = static_cast<const int8_t*>(w);
  if (w_is_int4) pick_mb<true>(q, s_a, wb, s_w, y, acc, M, N, K, st);
  else pick_mb<false>(q, s_a, wb, s_w, y, acc, M, N, K, st);
  return launch_status();
}

}  // namespace prism
