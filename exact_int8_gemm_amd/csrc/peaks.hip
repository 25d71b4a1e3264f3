// Measurement kernels: what the chip reaches on the two resources the GEMMs
// are bound by, measured with kernels of this library rather than taken
// from the data sheet.
//
//  * mfma_peak_kernel: each wave runs NACC independent chains of
//    v_mfma_i32_32x32x32_i8 on register operands (no memory traffic), two
//    workgroups per CU with 2 * WPS waves each, i.e. WPS waves per SIMD.
//    Ops per launch = workgroups x waves x iters x 16 x 65536.
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
