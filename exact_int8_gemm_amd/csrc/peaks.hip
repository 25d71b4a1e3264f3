// Measurement kernels: what the chip reaches on the two resources the GEMMs
// are bound by, measured with kernels of this library rather than taken
// from the data sheet.
//
//  * mfma_peak_kernel: each wave runs NACC independent chains of
//    v_mfma_i32_32x32x32_i8 on register operands (no memory traffic), two
//    workgroups per CU with 2 * WPS waves each, i.e. WPS waves per SIMD.
//    Ops per launch = workgroups x waves x iters x 16 x 65536.
//  * fold_probe_kernel: what one 32-k block of one 32 x 32 output tile costs
//    a SIMD in the block-scale GEMMs (one exact block sum, then one fp32
//    fold per output), on registers only, in five forms (see below).
//  * stream_read_kernel: reads a buffer once with 16-byte loads (8 in
//    flight per thread, grid-stride), eight 256-thread workgroups per CU,
//    and XORs what it read into one word per workgroup, so that no load can
//    be dropped and a test can check that every byte was read once.
#include "prism_internal.h"
#include "../../include/prism.h"

namespace prism {
namespace tiled {
namespace dma {
int device_cus();  // compute units of the current device (cached per device)
}  // namespace dma
}  // namespace tiled
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Pseudo-random fragment bytes over the whole int8 range (the MFMA's power
// draw, and so its clock, depends on the data): byte j (0..15) of operand
// `salt` in lane l is the top byte of (37 l + 101 j + 7919 salt + 13 seed)
// * 2654435761 (mod 2^32).
__device__ inline v4i fragment(int lane, int salt, int seed) {
  int d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t h = (uint32_t)(37 * lane + 101 * (4 * i + b) + 7919 * salt + 13 * seed) * 2654435761u;
      w |= (h >> 24) << (8 * b);
    }
    d[i] = (int)w;
  }
  return v4i{d[0], d[1], d[2], d[3]};
}

template <int WPS, int NACC>
__global__ __launch_bounds__(128 * WPS) void mfma_peak_kernel(int iters, int seed, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const v4i a0 = fragment(lane, 0, seed), b0 = fragment(lane, 1, seed);
  const v4i a1 = fragment(lane, 2, seed), b1 = fragment(lane, 3, seed);
  v16i acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = v16i{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 16 / NACC; ++r) {
#pragma unroll
      for (int i = 0; i < NACC; ++i)
        acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8((r & 1) ? a1 : a0, (r & 1) ? b1 : b0, acc[i], 0, 0, 0);
    }
  }
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += (uint32_t)acc[i][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Block-fold probe.  One workgroup of 8 waves per CU (2 waves per SIMD);
// each wave holds kFoldTiles tiles of 32 x 32 outputs and, per iteration,
// gives every tile one 32-k block:
//   mode 0: P = v_mfma_i32_32x32x32_i8(A, B_t, 0), f_t = fmaf((float)P, d_t,
//           f_t) -- the form of the block-scale GEMMs;
//   mode 1: P from two v_mfma_f32_32x32x16_f16 on the same values held as
//           f16 (the block sum is exact in fp32, so no convert), then the
//           same fold;
//   mode 2: the int8 MFMAs only (accumulating across iterations);
//   mode 3: the f16 MFMA pairs only (accumulating across iterations);
//   mode 4: the folds only, on fixed P.
// A alternates between two fragments per iteration; B_t and d_t differ per
// tile.  The f16 operands hold the int8 fragments' bytes 0-7 and 8-15 of
// each lane as the two 16-k halves, so every row and column pairs the same
// values in both forms: modes 0 and 1 give the same P and therefore the same
// bits, and so do modes 2 and 3 while the sums stay below 2^24 (iters <=
// 32).  Each thread writes the sum over its tiles and registers (fixed
// order) of f, or of the accumulators as fp32.
constexpr int kFoldTiles = 5;

template <int MODE>
__global__ __launch_bounds__(512) void fold_probe_kernel(int iters, float* __restrict__ out) {
  constexpr int T = kFoldTiles;
  const int lane = threadIdx.x & 63;
  v4i a[2], b[T];
  v8h ah[2][2], bh[T][2];
  float d[T];
  auto halves = [](const v4i x, v8h (&h)[2]) {
#pragma unroll
    for (int e = 0; e < 16; ++e) h[e / 8][e % 8] = (_Float16)(int8_t)((uint32_t)x[e / 4] >> (8 * (e % 4)));
  };
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[i] = fragment(lane, i, 0);
    halves(a[i], ah[i]);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    b[t] = fragment(lane, 2 + t, 0);
    halves(b[t], bh[t]);
    d[t] = 0.75f + (float)((lane * 7 + t * 13) & 63) * 0x1p-7f;
  }
  float f[T][16];
  v16i iacc[T];
  v16f facc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    iacc[t] = v16i{};
    facc[t] = v16f{};
#pragma unroll
    for (int r = 0; r < 16; ++r) f[t][r] = 0.0f;
  }
  auto block = [&](int i) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if constexpr (MODE == 0) {
        const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[t], v16i{}, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) f[t][r] = __builtin_fmaf((float)p[r], d[t], f[t][r]);
      } else if constexpr (MODE == 1) {
        v16f p = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i][0], bh[t][0], v16f{}, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i][1], bh[t][1], p, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) f[t][r] = __builtin_fmaf(p[r], d[t], f[t][r]);
      } else if constexpr (MODE == 2) {
        iacc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[t], iacc[t], 0, 0, 0);
      } else if constexpr (MODE == 3) {
        facc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i][0], bh[t][0], facc[t], 0, 0, 0);
        facc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i][1], bh[t][1], facc[t], 0, 0, 0);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) f[t][r] = __builtin_fmaf((float)(r + 16 * t + i), d[t], f[t][r]);
      }
    }
  };
  int it = 0;
  for (; it + 1 < iters; it += 2) {
    block(0);
    block(1);
  }
  if (it < iters) block(0);
  float s = 0.0f;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += MODE == 2 ? (float)iacc[t][r] : MODE == 3 ? facc[t][r] : f[t][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

constexpr int kReadThreads = 256, kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const v4i* __restrict__ p, int64_t n16,
                                                                   uint32_t* __restrict__ parts, int nparts) {
  __shared__ uint32_t red[kReadThreads / 64];
  const int64_t T = (int64_t)gridDim.x * kReadThreads;
  uint32_t x = 0;
  for (int64_t i0 = (int64_t)blockIdx.x * kReadThreads + threadIdx.x; i0 < n16; i0 += kReadUnroll * T) {
    v4i v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = i0 + u * T < n16 ? p[i0 + u * T] : v4i{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) parts[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
  if (blockIdx.x == 0)
    for (int b = (int)gridDim.x + threadIdx.x; b < nparts; b += kReadThreads) parts[b] = 0;
}

}  // namespace

int launch_peak_mfma(int64_t iters, int waves_per_simd, int seed, uint32_t* out, hipStream_t st) {
  const unsigned grid = 2u * (unsigned)tiled::dma::device_cus();
  switch (waves_per_simd) {
    case 1: mfma_peak_kernel<1, 8><<<grid, 128, 0, st>>>((int)iters, seed, out); break;
    case 2: mfma_peak_kernel<2, 8><<<grid, 256, 0, st>>>((int)iters, seed, out); break;
    case 4: mfma_peak_kernel<4, 4><<<grid, 512, 0, st>>>((int)iters, seed, out); break;
    default: return PRISM_ERR_INVALID_ARG;
  }
  return launch_status();
}

int launch_peak_fold(int mode, int64_t iters, float* out, hipStream_t st) {
  const unsigned grid = (unsigned)tiled::dma::device_cus();
  switch (mode) {
    case 0: fold_probe_kernel<0><<<grid, 512, 0, st>>>((int)iters, out); break;
    case 1: fold_probe_kernel<1><<<grid, 512, 0, st>>>((int)iters, out); break;
    case 2: fold_probe_kernel<2><<<grid, 512, 0, st>>>((int)iters, out); break;
    case 3: fold_probe_kernel<3><<<grid, 512, 0, st>>>((int)iters, out); break;
    case 4: fold_probe_kernel<4><<<grid, 512, 0, st>>>((int)iters, out); break;
    default: return PRISM_ERR_INVALID_ARG;
  }
  return launch_status();
}

int launch_peak_read(const void* buf, int64_t bytes, uint32_t* parts, int nparts, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  int64_t grid = (n16 + kReadThreads - 1) / kReadThreads;
  const int64_t cap = 8 * (int64_t)tiled::dma::device_cus();
  if (grid > cap) grid = cap;
  if (grid > nparts) grid = nparts;
  stream_read_kernel<<<(unsigned)grid, kReadThreads, 0, st>>>(static_cast<const v4i*>(buf), n16, parts, nparts);
  return launch_status();
}

}  // namespace prism
