// Ping-pong schedule of the int8 tiled GEMM (output tiles of 256 rows by BN =
// 192, 256 or 320 columns, eight waves, direct-to-LDS copies as in
// gemm_dma_kernel).
//
// The exact int32 sums of the StartLux-Prism README ("How it works") need a
// dense int8 contraction at large M; this kernel keeps the matrix cores of a
// CU busy while its own operand traffic is in flight.  The eight waves form
// two groups of four; wave w and wave w + 4 share a SIMD.  Group 0 owns the
// left BN / 2 columns of the tile and group 1 the right BN / 2, each wave a
// 64 x BN / 2 block of 2 x BN / 64 MFMA tiles of 32 x 32.
//
// Time is cut into phases by workgroup barriers.  In every phase one group
// runs the MFMAs of KSP 32-k steps from registers while the other group
// reads its fragments of the next KSP steps from LDS (and, once per stage,
// issues its share of the global -> LDS copies of a later stage); in the
// next phase the roles swap.  Group 1 starts one barrier late, so the two
// waves of a SIMD alternate and the MFMA unit always has queued work.
//
// Stages are BK bytes of k for all 512 rows (256 of A, 256 of B) in a ring
// of RING LDS buffers.  Both groups issue the copies of stage s + RING - 1
// in their first read phase of stage s, into the buffer of stage s - 1,
// which both groups finished reading before that phase's barrier.  Before
// the barrier that precedes the first read of stage s + 1 every wave waits
// (s_waitcnt vmcnt) for its own copies of that stage; the RING - 2 younger
// stages may stay in flight.  LDS layout, swizzle and out-of-range zeros are
// those of gemm_dma_kernel.
#pragma once

#include "gemm_tiled_kernels.h"

namespace prism {
namespace tiled {
namespace dma {

// Tile and k-split of this workgroup: as tile_of_split, but the tiles of an
// XCD's range are walked in groups of kGroupCols tile columns (column-major
// inside a group), so the workgroups that run together on one XCD share a
// few weight panels and many activation panels in its L2.  Measured on
// MI355X at M = 8192, N = K = 5120: 261 us against 280 us for groups of 8
// tile rows.
__device__ inline void tile_of_split_cols(int tiles_m, int tiles_n, int splits, int& tm, int& tn, int& split) {
  const int G = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  const int xcd = b % 8, r = b / 8;
  const int base = G / 8, rem = G % 8;
  const int id = xcd * base + min(xcd, rem) + r;
  const int tile = id / splits;
  split = id - tile * splits;
  constexpr int kGroupCols = 4;
  const int per_group = kGroupCols * tiles_m;
  const int grp = tile / per_group;
  const int first = grp * kGroupCols;
  const int gn = min(tiles_n - first, kGroupCols);
  const int in = tile - grp * per_group;
  tn = first + in % gn;
  tm = in / gn;
}

// Workgroup barrier that the compiler may not move memory accesses across.
__device__ inline void pp_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt lgkmcnt(0), no wait on vmcnt or expcnt (gfx9 encoding).
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int BK, int RING, int BN = 256, int KSP = 2>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(const int8_t* __restrict__ q, const float* __restrict__ s_a,
                                                        const int8_t* __restrict__ w, const float* __restrict__ s_w,
                                                        float* __restrict__ y, int32_t* __restrict__ acc_out, int M,
                                                        int N, int K, int tiles_m, int tiles_n, int splits) {
  constexpr int BM = 256;
  using C = Cfg<BM, BN, BK, 4, 2, RING>;
  constexpr int P = BK / (32 * KSP);  // read/compute phase pairs per stage (KSP 32-k steps each)
  constexpr int TM = 2, TN = BN / 64;
  static_assert(C::kNW == 8 && C::kPerWaveA * 8 == C::kCopiesA, "eight waves");
  __shared__ __attribute__((aligned(1024))) int8_t lds[RING * C::kStage];

  int tm, tn, split;
  tile_of_split_cols(tiles_m, tiles_n, splits, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave >> 2, wm = wave & 3;

  const int nk = (K + BK - 1) / BK;
  const int kb = (int)((int64_t)split * nk / splits), ke = (int)((int64_t)(split + 1) * nk / splits);
  const int kend = ke * BK < K ? ke * BK : K;

  // Copy sources of this wave (as in gemm_dma_kernel).
  const v4i ra = rsrc_words(q + (size_t)m0 * (size_t)K, (int64_t)(M - m0) * K);
  const v4i rb = rsrc_words(w + (size_t)n0 * (size_t)K, (int64_t)(N - n0) * K);
  // The k offset of a lane's chunk (chunk * 16) is recomputed at each issue
  // from the lane and the copy index instead of being kept per copy: a few
  // VALU operations in a read phase, against one register per copy.
  auto chunk_of = [&](int copy) __attribute__((always_inline)) {
    return (lane % C::kChunks) ^ C::swz(copy * C::kRowsPerCopy + lane / C::kChunks);
  };
  uint32_t off[C::kPerWave];
#pragma unroll
  for (int s = 0; s < C::kPerWave; ++s) {
    const bool isA = s < C::kPerWaveA;
    const int copy = isA ? wave * C::kPerWaveA + s : wave * C::kPerWaveB + (s - C::kPerWaveA);
    const int row = copy * C::kRowsPerCopy + lane / C::kChunks;
    const bool valid = isA ? (m0 + row < M) : (n0 + row < N);
    off[s] = valid ? (uint32_t)(row * K + chunk_of(copy) * 16) : kOutOfRange;
  }
  auto issue = [&](int buf, int stage) __attribute__((always_inline)) {
    const int k0 = stage * BK;
#pragma unroll
    for (int s = 0; s < C::kPerWave; ++s) {
      const bool isA = s < C::kPerWaveA;
      const int copy = isA ? wave * C::kPerWaveA + s : wave * C::kPerWaveB + (s - C::kPerWaveA);
      const uint32_t o = (k0 + chunk_of(copy) * 16 < kend) ? off[s] + (uint32_t)k0 : kOutOfRange;
      const int8_t* dst = lds + buf * C::kStage + (isA ? 0 : BM * BK) + copy * 1024;
      copy_to_lds(isA ? ra : rb, lds_addr(dst), o);
    }
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

  const int rl = lane & 31;
  const int sw = C::swz(rl);
  const int arow = (wm * 64 + rl) * BK;
  const int brow = (BM + grp * (BN / 2) + rl) * BK;
  v4i af[TM][KSP], bf[TN][KSP];
  // Fragments of the (32 KSP)-k slice `half` of the stage in buffer `buf`:
  // logical chunk 2 (KSP half + ks) + lane / 32 of row (lane % 32) of each
  // 32-row tile.
  auto read = [&](int buf, int half) __attribute__((always_inline)) {
    const int8_t* base = lds + buf * C::kStage;
#pragma unroll
    for (int ks = 0; ks < KSP; ++ks) {
      const int c = ((2 * (KSP * half + ks) + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i][ks] = *reinterpret_cast<const v4i*>(base + arow + i * 32 * BK + c);
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j][ks] = *reinterpret_cast<const v4i*>(base + brow + j * 32 * BK + c);
    }
  };
  auto mma = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KSP; ++ks)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i][ks], bf[j][ks], acc[i][j], 0, 0, 0);
  };

  // Stage count padded to a multiple of the ring: padded stages read zeros.
  const int nkr = (ke - kb + RING - 1) / RING * RING;
#pragma unroll
  for (int r = 0; r < RING - 1; ++r) issue(r, kb + r);
  wait_vmcnt<(RING - 2) * C::kPerWave>();
  pp_barrier();
  if (grp == 1) pp_barrier();  // group 1 runs one phase behind group 0
  __builtin_amdgcn_sched_barrier(0);

  for (int u = 0; u < nkr; u += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
#pragma unroll
      for (int h = 0; h < P; ++h) {
        // read phase of slice h of stage u + r (buffer r)
        if (h == 0) issue((r + RING - 1) % RING, kb + u + r + RING - 1);
        read(r, h);
        wait_lgkm0();
        if (h == P - 1 && grp == 1) wait_vmcnt<(RING - 2) * C::kPerWave>();
        __builtin_amdgcn_sched_barrier(0);
        pp_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // compute phase
        mma();
        if (h == P - 1 && grp == 0) wait_vmcnt<(RING - 2) * C::kPerWave>();
        __builtin_amdgcn_sched_barrier(0);
        pp_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (grp == 0) pp_barrier();  // matches group 1's extra barrier at the start
  wait_vmcnt<0>();             // no copy may land in LDS after the workgroup ends

  const int mb = m0 + wm * 64, nb = n0 + grp * (BN / 2);
  if (splits > 1) {
    int32_t* yi = reinterpret_cast<int32_t*>(y);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = nb + j * 32 + rl;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mb + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          if (m < M)
            __hip_atomic_fetch_add(yi + (size_t)m * (size_t)N + (size_t)n, acc[i][j][r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    return;
  }
  // The tile's row and column scales, loaded once into LDS: reading them per
  // element from global memory inside the store loop (32 row scales per
  // lane) cost about 44 of 270 us at M = 8192, N = K = 5120.
  __shared__ float sa_l[BM], sw_l[BN];
  for (int t = threadIdx.x; t < BM + BN; t += 512) {
    if (t < BM) sa_l[t] = m0 + t < M ? s_a[m0 + t] : 0.0f;
    else sw_l[t - BM] = n0 + t - BM < N ? s_w[n0 + t - BM] : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = nb + j * 32 + rl;
    if (n >= N) continue;
    const float swn = sw_l[n - n0];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < M) {
          const int a = acc[i][j][r];
          const size_t o = (size_t)m * (size_t)N + (size_t)n;
          if (acc_out) acc_out[o] = a;
          const float t = (float)a * sa_l[m - m0];
          y[o] = t * swn;
        }
      }
    }
  }
}

template <int BK, int RING, int BN = 256, int KSP = 2>
void launch_pp(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc, int M,
               int N, int K, hipStream_t st, int splits = 1) {
  const int tiles_m = (M + 255) / 256, tiles_n = (N + BN - 1) / BN;
  const int64_t total = (int64_t)M * N;
  if (splits > 1)
    zero_kernel<<<(unsigned)((total + 1023) / 1024), 256, 0, st>>>(reinterpret_cast<int32_t*>(y), total);
  gemm_pp_kernel<BK, RING, BN, KSP><<<(unsigned)(tiles_m * tiles_n * splits), 512, 0, st>>>(q, s_a, w, s_w, y, acc, M, N, K,
                                                                                   tiles_m, tiles_n, splits);
  if (splits > 1) launch_finalize(y, acc, s_a, s_w, M, N, st);
}

}  // namespace dma
}  // namespace tiled
}  // namespace prism
