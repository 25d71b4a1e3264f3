// LDS-tiled GEMMs for M > 64: W8A8 and W4A8 with per-channel scales, and
// W8A8 with fp16 scales per 32-k block.
//
// The exact int32 sums of the StartLux-Prism README ("Why StartLux-Prism",
// "How it works") are computed with v_mfma_i32_32x32x32_i8.  One workgroup
// owns a BM x BN output tile and walks K in stages of BK = 128 bytes:
//
//  * stage k+1 is fetched from HBM into registers with 16-byte loads while
//    stage k is multiplied out of LDS (two LDS buffers, one barrier per
//    stage);
//  * LDS rows are BK + 16 bytes apart, which puts the 16-byte operand reads
//    of 8 (or 16) consecutive lanes into distinct 16-byte bank groups;
//  * 4-bit weights are unpacked once per tile on their way into LDS (nibble
//    moved to the top of a byte, i.e. 16 * w as int8), so the inner loop is
//    the same as for int8 weights and the accumulator is shifted right by 4;
//  * MFMA lane layout (32x32x32): lane l supplies row (l % 32) of the A tile
//    and column (l % 32) of the B tile, with k-group l / 32; both operands use
//    the same lane -> k assignment, so the integer sum is the plain dot
//    product.  The int32 result of lane l, register r sits at row
//    8 * (r / 4) + 4 * (l / 32) + (r % 4), column l % 32;
//  * workgroups are renumbered so that each of the 8 XCDs (which receive
//    workgroups round-robin) runs a contiguous range of tiles, walked in
//    groups of 8 tile rows so that neighbouring tiles share operand panels
//    in that XCD's L2.
//
// Epilogues, per element and in a fixed order:
//   per channel: y = ((float)acc * s_a[m]) * s_w[n]
//   per block:   f = +0; for b ascending f = fmaf((float)P_b, (float)d[n][b], f);
//                y = f * s_a[m]
#include "prism_internal.h"
#include "../../include/prism.h"

namespace prism {
namespace {

constexpr int BK = 128;
constexpr int kLdsStride = BK + 16;

__device__ inline v4i load16(const int8_t* p) { return *reinterpret_cast<const v4i*>(p); }

__device__ inline void unpack_w4(const v4i p, v4i& lo, v4i& hi) {
  int o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = (uint32_t)p[j];
    const uint32_t L = (u << 4) & 0xF0F0F0F0u;
    const uint32_t H = u & 0xF0F0F0F0u;
    o[2 * j] = (int)__builtin_amdgcn_perm(H, L, 0x05010400u);
    o[2 * j + 1] = (int)__builtin_amdgcn_perm(H, L, 0x07030602u);
  }
  lo = v4i{o[0], o[1], o[2], o[3]};
  hi = v4i{o[4], o[5], o[6], o[7]};
}

// Tile index of this workgroup: XCD-contiguous renumbering, then grouped
// row-major order over the tile grid.
__device__ inline void tile_of(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int G = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  const int xcd = b % 8, r = b / 8;
  const int base = G / 8, rem = G % 8;
  const int id = xcd * base + min(xcd, rem) + r;
  constexpr int kGroup = 8;
  const int per_group = kGroup * tiles_n;
  const int grp = id / per_group;
  const int first = grp * kGroup;
  const int gm = min(tiles_m - first, kGroup);
  const int in = id - grp * per_group;
  tm = first + in % gm;
  tn = in / gm;
}

// Global -> register -> LDS staging of one BK slice of the A (activation)
// and B (weight) tiles.
template <int BM, int BN, int NT, bool W4>
struct Stager {
  static constexpr int kAChunks = BM * (BK / 16) / NT;
  static constexpr int kBChunks = W4 ? BN * (BK / 32) / NT : BN * (BK / 16) / NT;
  static_assert(BM * (BK / 16) % NT == 0, "A tile chunks must divide among threads");
  static_assert((W4 ? BN * (BK / 32) : BN * (BK / 16)) % NT == 0, "B tile chunks must divide among threads");

  v4i ra[kAChunks];
  v4i rb[kBChunks];

  __device__ inline void load(const int8_t* __restrict__ q, const int8_t* __restrict__ w, int m0, int n0, int k0,
                              int M, int N, int K) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / (BK / 16), c = idx % (BK / 16);
      const int m = m0 + r, k = k0 + c * 16;
      ra[i] = (m < M && k < K) ? load16(q + (size_t)m * (size_t)K + k) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int idx = tid + i * NT;
      if (W4) {
        const int r = idx / (BK / 32), c = idx % (BK / 32);
        const int n = n0 + r, k = k0 + c * 32;
        rb[i] = (n < N && k < K) ? load16(w + (size_t)n * (size_t)(K / 2) + k / 2) : v4i{0, 0, 0, 0};
      } else {
        const int r = idx / (BK / 16), c = idx % (BK / 16);
        const int n = n0 + r, k = k0 + c * 16;
        rb[i] = (n < N && k < K) ? load16(w + (size_t)n * (size_t)K + k) : v4i{0, 0, 0, 0};
      }
    }
  }

  __device__ inline void store(int8_t* lds) const {
    const int tid = threadIdx.x;
    int8_t* sa = lds;
    int8_t* sb = lds + BM * kLdsStride;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / (BK / 16), c = idx % (BK / 16);
      *reinterpret_cast<v4i*>(sa + r * kLdsStride + c * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int idx = tid + i * NT;
      if (W4) {
        const int r = idx / (BK / 32), c = idx % (BK / 32);
        v4i lo, hi;
        unpack_w4(rb[i], lo, hi);
        *reinterpret_cast<v4i*>(sb + r * kLdsStride + c * 32) = lo;
        *reinterpret_cast<v4i*>(sb + r * kLdsStride + c * 32 + 16) = hi;
      } else {
        const int r = idx / (BK / 16), c = idx % (BK / 16);
        *reinterpret_cast<v4i*>(sb + r * kLdsStride + c * 16) = rb[i];
      }
    }
  }
};

template <int BM, int BN, int WM, int WN, bool W4>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tiled_kernel(const int8_t* __restrict__ q,
                                                                  const float* __restrict__ s_a,
                                                                  const int8_t* __restrict__ w,
                                                                  const float* __restrict__ s_w,
                                                                  float* __restrict__ y,
                                                                  int32_t* __restrict__ acc_out, int M, int N,
                                                                  int K, int tiles_m, int tiles_n) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM * 32 == WTM && TN * 32 == WTN, "wave tile must be a multiple of 32x32");
  __shared__ __attribute__((aligned(16))) int8_t lds[2][(BM + BN) * kLdsStride];

  int tm, tn;
  tile_of(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

  Stager<BM, BN, NT, W4> st;
  const int nk = (K + BK - 1) / BK;
  st.load(q, w, m0, n0, 0, M, N, K);
  st.store(lds[0]);
  __syncthreads();

  const int rl = lane & 31, kg = (lane >> 5) * 16;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) st.load(q, w, m0, n0, (kt + 1) * BK, M, N, K);
    const int8_t* sa = lds[cur] + (wm * WTM + rl) * kLdsStride + kg;
    const int8_t* sb = lds[cur] + (BM + wn * WTN + rl) * kLdsStride + kg;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      v4i af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const v4i*>(sa + i * 32 * kLdsStride + ks * 32);
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const v4i*>(sb + j * 32 * kLdsStride + ks * 32);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) st.store(lds[cur ^ 1]);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + wn * WTN + j * 32 + rl;
    if (n >= N) continue;
    const float sw = s_w[n];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < M) {
          int a = acc[i][j][r];
          if (W4) a >>= 4;  // exact: the sum is a multiple of 16
          const size_t o = (size_t)m * (size_t)N + (size_t)n;
          if (acc_out) acc_out[o] = a;
          const float t = (float)a * s_a[m];
          y[o] = t * sw;
        }
      }
    }
  }
}

__device__ inline float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_blockscale_kernel(const int8_t* __restrict__ q,
                                                                       const float* __restrict__ s_a,
                                                                       const int8_t* __restrict__ w,
                                                                       const uint16_t* __restrict__ d,
                                                                       float* __restrict__ y,
                                                                       int32_t* __restrict__ partials, int M,
                                                                       int N, int K, int tiles_m, int tiles_n) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int KS = BK / 32;  // 32-k blocks per stage
  static_assert(TM * 32 == WTM && TN * 32 == WTN, "wave tile must be a multiple of 32x32");
  __shared__ __attribute__((aligned(16))) int8_t lds[2][(BM + BN) * kLdsStride];

  int tm, tn;
  tile_of(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int rl = lane & 31, kg = (lane >> 5) * 16;
  const int NB = K / 32;

  float f[TM][TN][16];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) f[i][j][r] = 0.0f;

  // This lane's output columns and their block-scale rows.
  int ncol[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) ncol[j] = n0 + wn * WTN + j * 32 + rl;

  Stager<BM, BN, NT, false> st;
  const int nk = (K + BK - 1) / BK;
  st.load(q, w, m0, n0, 0, M, N, K);
  st.store(lds[0]);
  __syncthreads();

  const v16i zero = v16i{};
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    float dv[TN][KS];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int b = kt * KS + ks;
        dv[j][ks] = (ncol[j] < N && b < NB) ? half_bits_to_float(d[(size_t)ncol[j] * (size_t)NB + b]) : 0.0f;
      }
    if (kt + 1 < nk) st.load(q, w, m0, n0, (kt + 1) * BK, M, N, K);
    const int8_t* sa = lds[cur] + (wm * WTM + rl) * kLdsStride + kg;
    const int8_t* sb = lds[cur] + (BM + wn * WTN + rl) * kLdsStride + kg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int b = kt * KS + ks;
      if (b >= NB) break;  // uniform over the workgroup
      v4i af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const v4i*>(sa + i * 32 * kLdsStride + ks * 32);
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const v4i*>(sb + j * 32 * kLdsStride + ks * 32);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], zero, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) f[i][j][r] = __builtin_fmaf((float)p[r], dv[j][ks], f[i][j][r]);
          if (partials) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int m = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
              if (m < M && ncol[j] < N)
                partials[((size_t)m * (size_t)N + (size_t)ncol[j]) * (size_t)NB + b] = p[r];
            }
          }
        }
    }
    if (kt + 1 < nk) st.store(lds[cur ^ 1]);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if (ncol[j] >= N) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < M) y[(size_t)m * (size_t)N + (size_t)ncol[j]] = f[i][j][r] * s_a[m];
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, bool W4>
void launch_tiled(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc,
                  int M, int N, int K, hipStream_t st) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  gemm_tiled_kernel<BM, BN, WM, WN, W4>
      <<<(unsigned)(tiles_m * tiles_n), 64 * WM * WN, 0, st>>>(q, s_a, w, s_w, y, acc, M, N, K, tiles_m, tiles_n);
}

template <bool W4>
void pick_tile(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc, int M,
               int N, int K, hipStream_t st) {
  // Large tiles when they still give every CU at least one tile.
  const int64_t big = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  if (big >= 256) launch_tiled<256, 256, 2, 4, W4>(q, s_a, w, s_w, y, acc, M, N, K, st);
  else launch_tiled<128, 128, 2, 2, W4>(q, s_a, w, s_w, y, acc, M, N, K, st);
}

}  // namespace

int launch_gemm_tiled(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w, float* y,
                      int32_t* acc, int M, int N, int K, hipStream_t st) {
  const int8_t* wb = static_cast<const int8_t*>(w);
  if (w_is_int4) pick_tile<true>(q, s_a, wb, s_w, y, acc, M, N, K, st);
  else pick_tile<false>(q, s_a, wb, s_w, y, acc, M, N, K, st);
  return launch_status();
}

int launch_gemm_blockscale(const int8_t* q, const float* s_a, const int8_t* w, const uint16_t* d, float* y,
                           int32_t* partials, int M, int N, int K, hipStream_t st) {
  constexpr int BM = 128, BN = 128, WM = 2, WN = 2;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  gemm_blockscale_kernel<BM, BN, WM, WN>
      <<<(unsigned)(tiles_m * tiles_n), 64 * WM * WN, 0, st>>>(q, s_a, w, d, y, partials, M, N, K, tiles_m, tiles_n);
  return launch_status();
}

}  // namespace prism
