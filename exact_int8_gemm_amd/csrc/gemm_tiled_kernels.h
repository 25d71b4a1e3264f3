// LDS-tiled GEMM kernels for gfx950: W8A8 and W4A8 with per-channel scales,
// and W8A8 with fp16 scales per 32-k block.
//
// The exact int32 sums of the StartLux-Prism README ("Why StartLux-Prism",
// "How it works") are computed with v_mfma_i32_32x32x32_i8.  One workgroup
// owns a BM x BN output tile and walks K in stages of BK bytes:
//
//  * software pipeline: the 16-byte global loads of stage k+2 are issued
//    into one of two register sets while stage k is multiplied out of LDS
//    and stage k+1 waits in the other register set; stage k+1 is written to
//    the second LDS buffer at the end of the iteration, then one barrier.
//    A load therefore has about two stages of MFMA work to arrive;
//  * LDS rows are BK + 16 bytes apart, which puts the 16-byte operand reads
//    of 8 (or 16) consecutive lanes into distinct bank groups;
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
#pragma once

#include <type_traits>

#include "lds_copy.h"
#include "prism_internal.h"

namespace prism {
namespace tiled {

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

// The same for 8 packed bytes (16 nibbles) -> one 16-byte fragment.
__device__ inline v4i unpack_w4_8(const v2i p) {
  int o[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t u = (uint32_t)p[j];
    const uint32_t L = (u << 4) & 0xF0F0F0F0u;
    const uint32_t H = u & 0xF0F0F0F0u;
    o[2 * j] = (int)__builtin_amdgcn_perm(H, L, 0x05010400u);
    o[2 * j + 1] = (int)__builtin_amdgcn_perm(H, L, 0x07030602u);
  }
  return v4i{o[0], o[1], o[2], o[3]};
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

// Tile and k-split of this workgroup: workgroup ids are split-major inside
// each XCD's range, so the splits of one tile run on the same XCD.
__device__ inline void tile_of_split(int tiles_m, int tiles_n, int splits, int& tm, int& tn, int& split) {
  const int G = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  const int xcd = b % 8, r = b / 8;
  const int base = G / 8, rem = G % 8;
  const int id = xcd * base + min(xcd, rem) + r;
  const int tile = id / splits;
  split = id - tile * splits;
  constexpr int kGroup = 8;
  const int per_group = kGroup * tiles_n;
  const int grp = tile / per_group;
  const int first = grp * kGroup;
  const int gm = min(tiles_m - first, kGroup);
  const int in = tile - grp * per_group;
  tm = first + in % gm;
  tn = in / gm;
}

__device__ inline float half_bits_to_float(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }


// Buffer resource over `bytes` bytes from `base` (raw, stride 0); accesses at
// offsets past the end return zero.  Clamped below kOutOfRange.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < (int64_t)kOutOfRange - 1 ? bytes : (int64_t)kOutOfRange - 1;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// One BK slice of the A (activation) and B (weight) tiles, held in registers
// between its global loads and its LDS stores.  Loads are branch-free buffer
// loads: a row outside the matrix has an out-of-range base offset and a
// chunk past K is sent out of range, so both read zeros.
template <int BM, int BN, int BK, int NT, bool W4>
struct Stage {
  static constexpr int kSA = BK + 16;                 // LDS row stride (bytes)
  static constexpr int kCA = BK / 16;                 // 16-byte chunks per A row
  static constexpr int kCB = W4 ? BK / 32 : BK / 16;  // 16-byte global chunks per B row
  static constexpr int kNA = BM * kCA / NT;
  static constexpr int kNB = BN * kCB / NT;
  static_assert(BM * kCA % NT == 0 && BN * kCB % NT == 0, "tile chunks must divide among threads");

  v4i a[kNA];
  v4i b[kNB];
};

// Per-thread addressing of the stage loads and LDS stores, fixed for the
// whole tile.
template <int BM, int BN, int BK, int NT, bool W4>
struct StageAddr {
  using S = Stage<BM, BN, BK, NT, W4>;
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t oa[S::kNA], ob[S::kNB];  // byte offset of the chunk at k0 = 0 (or out of range)
  int ka[S::kNA], kb[S::kNB];       // k of the chunk at k0 = 0

  __device__ inline void init(const int8_t* q, const int8_t* w, int m0, int n0, int M, int N, int K) {
    const int tid = threadIdx.x;
    const int64_t wrow = W4 ? K / 2 : K;
    ra = make_rsrc(q + (size_t)m0 * (size_t)K, (int64_t)(M - m0) * K);
    rb = make_rsrc(w + (size_t)n0 * (size_t)wrow, (int64_t)(N - n0) * wrow);
#pragma unroll
    for (int i = 0; i < S::kNA; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / S::kCA, c = idx % S::kCA;
      ka[i] = c * 16;
      oa[i] = (m0 + r < M) ? (uint32_t)(r * K + c * 16) : kOutOfRange;
    }
#pragma unroll
    for (int i = 0; i < S::kNB; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / S::kCB, c = idx % S::kCB;
      kb[i] = W4 ? c * 32 : c * 16;
      ob[i] = (n0 + r < N) ? (uint32_t)(r * wrow + c * 16) : kOutOfRange;  // W4: 16 packed bytes = 32 k
    }
  }

  __device__ inline void load(S& s, int k0, int K) const {
#pragma unroll
    for (int i = 0; i < S::kNA; ++i) {
      const uint32_t off = (k0 + ka[i] < K) ? oa[i] + (uint32_t)k0 : kOutOfRange;
      s.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < S::kNB; ++i) {
      const uint32_t kb0 = W4 ? (uint32_t)(k0 / 2) : (uint32_t)k0;
      const uint32_t off = (k0 + kb[i] < K) ? ob[i] + kb0 : kOutOfRange;
      s.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
    }
  }

  __device__ inline void store(const S& s, int8_t* lds) const {
    const int tid = threadIdx.x;
    int8_t* sa = lds;
    int8_t* sb = lds + BM * S::kSA;
#pragma unroll
    for (int i = 0; i < S::kNA; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / S::kCA, c = idx % S::kCA;
      *reinterpret_cast<v4i*>(sa + r * S::kSA + c * 16) = s.a[i];
    }
#pragma unroll
    for (int i = 0; i < S::kNB; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / S::kCB, c = idx % S::kCB;
      if (W4) {
        v4i lo, hi;
        unpack_w4(s.b[i], lo, hi);
        *reinterpret_cast<v4i*>(sb + r * S::kSA + c * 32) = lo;
        *reinterpret_cast<v4i*>(sb + r * S::kSA + c * 32 + 16) = hi;
      } else {
        *reinterpret_cast<v4i*>(sb + r * S::kSA + c * 16) = s.b[i];
      }
    }
  }
};

template <int BM, int BN, int BK, int WM, int WN>
struct Geometry {
  static constexpr int kNT = 64 * WM * WN;
  static constexpr int kSA = BK + 16;
  static constexpr int kWTM = BM / WM, kWTN = BN / WN;
  static constexpr int kTM = kWTM / 32, kTN = kWTN / 32;
  static constexpr int kLds = (BM + BN) * kSA;  // bytes per LDS buffer
  static_assert(kTM * 32 == kWTM && kTN * 32 == kWTN, "wave tile must be a multiple of 32x32");
  static_assert(BK % 32 == 0, "stage depth must be a multiple of 32");
};

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Multiply-accumulate one LDS stage into acc.  The operand fragments of k-step
// ks+1 are read from LDS while the MFMAs of k-step ks run (one fragment read
// after each of the first MFMAs), so LDS latency hides behind matrix work.
template <int BM, int BN, int BK, int WM, int WN>
__device__ inline void mma_stage(const int8_t* lds, int wm, int wn, int lane,
                                 v16i (&acc)[Geometry<BM, BN, BK, WM, WN>::kTM][Geometry<BM, BN, BK, WM, WN>::kTN]) {
  using G = Geometry<BM, BN, BK, WM, WN>;
  constexpr int KS = BK / 32;
  constexpr int NF = G::kTM + G::kTN;  // fragments per k-step
  const int rl = lane & 31, kg = (lane >> 5) * 16;
  const int8_t* sa = lds + (wm * G::kWTM + rl) * G::kSA + kg;
  const int8_t* sb = lds + (BM + wn * G::kWTN + rl) * G::kSA + kg;
  v4i af[2][G::kTM], bf[2][G::kTN];
#pragma unroll
  for (int i = 0; i < G::kTM; ++i) af[0][i] = *reinterpret_cast<const v4i*>(sa + i * 32 * G::kSA);
#pragma unroll
  for (int j = 0; j < G::kTN; ++j) bf[0][j] = *reinterpret_cast<const v4i*>(sb + j * 32 * G::kSA);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1, nxt = cur ^ 1;
    if (ks + 1 < KS) {
#pragma unroll
      for (int i = 0; i < G::kTM; ++i)
        af[nxt][i] = *reinterpret_cast<const v4i*>(sa + i * 32 * G::kSA + (ks + 1) * 32);
#pragma unroll
      for (int j = 0; j < G::kTN; ++j)
        bf[nxt][j] = *reinterpret_cast<const v4i*>(sb + j * 32 * G::kSA + (ks + 1) * 32);
    }
#pragma unroll
    for (int i = 0; i < G::kTM; ++i)
#pragma unroll
      for (int j = 0; j < G::kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[cur][i], bf[cur][j], acc[i][j], 0, 0, 0);
    if (ks + 1 < KS) {
      // interleave: MFMA, fragment read, MFMA, fragment read, ..., then the rest of the MFMAs
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, G::kTM * G::kTN - NF, 0);
    }
  }
}

// splits > 1: as in the direct-to-LDS kernel below, workgroup (tile, split)
// sums one contiguous range of stages and adds its partial tile into y
// viewed as int32 (4-bit: each partial is a multiple of 16 on its own and is
// shifted back before the add, so the sum needs no further step).
template <int BM, int BN, int BK, int WM, int WN, bool W4, int OCC>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_tiled_kernel(const int8_t* __restrict__ q,
                                                                       const float* __restrict__ s_a,
                                                                       const int8_t* __restrict__ w,
                                                                       const float* __restrict__ s_w,
                                                                       float* __restrict__ y,
                                                                       int32_t* __restrict__ acc_out, int M, int N,
                                                                       int K, int tiles_m, int tiles_n, int splits) {
  using G = Geometry<BM, BN, BK, WM, WN>;
  __shared__ __attribute__((aligned(16))) int8_t lds[2][G::kLds];

  int tm, tn, split;
  tile_of_split(tiles_m, tiles_n, splits, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  v16i acc[G::kTM][G::kTN];
#pragma unroll
  for (int i = 0; i < G::kTM; ++i)
#pragma unroll
    for (int j = 0; j < G::kTN; ++j) acc[i][j] = v16i{};

  StageAddr<BM, BN, BK, G::kNT, W4> ad;
  ad.init(q, w, m0, n0, M, N, K);
  Stage<BM, BN, BK, G::kNT, W4> s0, s1;
  // This split's stages [kb, ke); loads are bounded by kend, so stages past
  // ke read zeros instead of another split's k.
  const int nk = (K + BK - 1) / BK;
  const int kb = (int)((int64_t)split * nk / splits), ke = (int)((int64_t)(split + 1) * nk / splits);
  const int kend = ke * BK < K ? ke * BK : K;
  auto mma = [&](int buf) __attribute__((always_inline)) { mma_stage<BM, BN, BK, WM, WN>(lds[buf], wm, wn, lane, acc); };

  // Pipeline: stage k is in LDS buffer k % 2, stage k+1 waits in a register
  // set, stage k+2 is being loaded into the other set.  The stage count is
  // rounded up to even: stages at or past kend load as zeros (every chunk is
  // out of range), so the loop needs no tail and no conditions.
  ad.load(s0, kb * BK, kend);
  ad.load(s1, (kb + 1) * BK, kend);
  ad.store(s0, lds[0]);
  __syncthreads();
  // The scheduling barriers keep the global loads of a stage ahead of the
  // MFMAs (so they have two stages of work to arrive) and the LDS writes of
  // the waiting stage behind them.
  for (int k = kb; k < ke; k += 2) {
    ad.load(s0, (k + 2) * BK, kend);
    __builtin_amdgcn_sched_barrier(0);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    ad.store(s1, lds[1]);
    __syncthreads();
    ad.load(s1, (k + 3) * BK, kend);
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
    ad.store(s0, lds[0]);
    __syncthreads();
  }

  const int rl = lane & 31;
  // Register r of tile (i, j) holds row mb + 32 i + (r / 4) * 8 + r % 4 and
  // column nb + 32 j; interior tiles store without per-element bounds checks.
  const int mb = m0 + wm * G::kWTM + (lane >> 5) * 4, nb = n0 + wn * G::kWTN + rl;
  const bool full = m0 + BM <= M && n0 + BN <= N;
  if (splits > 1) {
    int32_t* yi = reinterpret_cast<int32_t*>(y);
    auto partial = [&](auto checked) __attribute__((always_inline)) {
      constexpr bool CHK = decltype(checked)::value;
#pragma unroll
      for (int j = 0; j < G::kTN; ++j) {
        const int n = nb + j * 32;
        if (CHK && n >= N) continue;
#pragma unroll
        for (int i = 0; i < G::kTM; ++i) {
          const int mr = mb + i * 32;
          int32_t* p = yi + (size_t)mr * (size_t)N + (size_t)n;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int dr = (r >> 2) * 8 + (r & 3);
            if (CHK && mr + dr >= M) continue;
            const int a = W4 ? (acc[i][j][r] >> 4) : acc[i][j][r];  // exact: each 4-bit partial is a multiple of 16
            __hip_atomic_fetch_add(p + (size_t)dr * (size_t)N, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    };
    if (full) partial(std::false_type{});
    else partial(std::true_type{});
    return;
  }
  // The tile's row and column scales, loaded once into LDS instead of per
  // element inside the store loop (as in the direct-to-LDS kernels).
  __shared__ __attribute__((aligned(16))) float sa_l[BM];
  __shared__ float sw_l[BN];
  for (int t = threadIdx.x; t < BM + BN; t += G::kNT) {
    if (t < BM) sa_l[t] = m0 + t < M ? s_a[m0 + t] : 0.0f;
    else sw_l[t - BM] = n0 + t - BM < N ? s_w[n0 + t - BM] : 0.0f;
  }
  __syncthreads();
  auto epilogue = [&](auto with_acc, auto checked) __attribute__((always_inline)) {
    constexpr bool ACC = decltype(with_acc)::value, CHK = decltype(checked)::value;
#pragma unroll
    for (int i = 0; i < G::kTM; ++i) {
      const int mr = mb + i * 32;
      float sa[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4f v = *reinterpret_cast<const v4f*>(sa_l + (mr - m0) + 8 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) sa[4 * g + e] = v[e];
      }
#pragma unroll
      for (int j = 0; j < G::kTN; ++j) {
        const int n = nb + j * 32;
        if (CHK && n >= N) continue;
        const float sw = sw_l[n - n0];
        float* yp = y + (size_t)mr * (size_t)N + (size_t)n;
        int32_t* ap = ACC ? acc_out + (size_t)mr * (size_t)N + (size_t)n : nullptr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dr = (r >> 2) * 8 + (r & 3);
          if (CHK && mr + dr >= M) continue;
          int a = acc[i][j][r];
          if (W4) a >>= 4;  // exact: the sum is a multiple of 16
          if constexpr (ACC) ap[(size_t)dr * (size_t)N] = a;
          const float t = (float)a * sa[r];
          yp[(size_t)dr * (size_t)N] = t * sw;
        }
      }
    }
  };
  if (acc_out) {
    if (full) epilogue(std::true_type{}, std::false_type{});
    else epilogue(std::true_type{}, std::true_type{});
  } else {
    if (full) epilogue(std::false_type{}, std::false_type{});
    else epilogue(std::false_type{}, std::true_type{});
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS pipeline (int8 weights).
//
// Stages of BK bytes of k are copied from HBM straight into an LDS ring of
// RING buffers by buffer_load_dwordx4 ... lds (no register staging): lane i
// of a wave-wide copy writes 16 bytes at LDS base + 16 i, so one copy moves
// 1024 / BK rows of BK bytes.  With BK = 128 every row of a copy is one full
// 128-byte line, which halves the number of L2 requests compared with
// 64-byte row pieces (the L2 request rate is what bounds this kernel).
// Rows are BK bytes apart in LDS and the 16-byte chunks of row r are stored
// in the order c ^ swz(r), chosen so that the fragment reads of 16
// consecutive lanes (16 consecutive rows, same chunk) fall in 16 distinct
// 16-byte groups of the 64 LDS banks.  Out-of-range copies (rows past M or N,
// k past K) write zeros.
//
// Iteration k: wait until this wave's copies of stage k have landed (the
// copies of the RING - 2 later stages may still be in flight), barrier (all
// waves' copies of stage k landed, all waves done with stage k - 1), start
// the copies of stage k + RING - 1 into the buffer of stage k - 1, then run
// the MFMAs of stage k.  Copies are always issued, also for stages past K
// (they write zeros and are never read), so the number of copies in flight
// at each wait is a constant.
namespace dma {

template <int BM, int BN, int BK, int WM, int WN, int RING>
struct Cfg {
  static constexpr int kNW = WM * WN;
  static constexpr int kNT = 64 * kNW;
  static constexpr int kChunks = BK / 16;          // 16-byte chunks per row
  static constexpr int kRowsPerCopy = 1024 / BK;   // rows per wave-wide copy
  static constexpr int kRowsPerWindow = 256 / BK;  // rows per 256-byte bank window
  static constexpr int kCopiesA = BM * BK / 1024;  // copies per stage
  static constexpr int kCopiesB = BN * BK / 1024;
  static constexpr int kPerWaveA = kCopiesA / kNW;
  static constexpr int kPerWaveB = kCopiesB / kNW;
  static constexpr int kPerWave = kPerWaveA + kPerWaveB;
  static constexpr int kStage = (BM + BN) * BK;
  static constexpr int kWTM = BM / WM, kWTN = BN / WN;
  static constexpr int kTM = kWTM / 32, kTN = kWTN / 32;
  static_assert(BK == 64 || BK == 128, "stage depth");
  static_assert(kCopiesA % kNW == 0 && kCopiesB % kNW == 0, "copies must divide among waves");
  static_assert(kTM * 32 == kWTM && kTN * 32 == kWTN, "wave tile must be a multiple of 32x32");
  static_assert(RING >= 2 && RING <= 4, "ring depth");
  static_assert(RING * kStage <= 160 * 1024, "LDS ring exceeds 160 KiB");
  static_assert((RING - 2) * kPerWave < 64, "vmcnt range");
  __device__ static int swz(int row) { return (row / kRowsPerWindow) % kChunks; }
};

// splits > 1: workgroup (tile, split) sums the split-th contiguous range of
// stages and adds its int32 partial tile into y viewed as int32 (zeroed
// before; the fp32 epilogue runs afterwards in finalize_kernel).  Integer
// addition is exact and associative, so the result does not depend on the
// order in which the partial tiles arrive.
template <int BM, int BN, int BK, int WM, int WN, int RING, int OCC>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_dma_kernel(const int8_t* __restrict__ q,
                                                                     const float* __restrict__ s_a,
                                                                     const int8_t* __restrict__ w,
                                                                     const float* __restrict__ s_w,
                                                                     float* __restrict__ y,
                                                                     int32_t* __restrict__ acc_out, int M, int N,
                                                                     int K, int tiles_m, int tiles_n, int splits) {
  using C = Cfg<BM, BN, BK, WM, WN, RING>;
  // Separate buffers (not one indexed array), so that every copy and every
  // read names its buffer statically.
  __shared__ __attribute__((aligned(1024))) int8_t lds0[C::kStage];
  __shared__ __attribute__((aligned(1024))) int8_t lds1[C::kStage];
  __shared__ __attribute__((aligned(1024))) int8_t lds2[RING > 2 ? C::kStage : 16];
  __shared__ __attribute__((aligned(1024))) int8_t lds3[RING > 3 ? C::kStage : 16];

  int tm, tn, split;
  tile_of_split(tiles_m, tiles_n, splits, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // This split's stages [kb, ke); copies are bounded by kend, so the padded
  // stages of the ring (past ke) read as zeros instead of other splits' k.
  const int nk = (K + BK - 1) / BK;
  const int kb = (int)((int64_t)split * nk / splits), ke = (int)((int64_t)(split + 1) * nk / splits);
  const int kend = ke * BK < K ? ke * BK : K;

  // Copy sources: this lane's row and chunk in each of the wave's copies.
  const v4i ra = rsrc_words(q + (size_t)m0 * (size_t)K, (int64_t)(M - m0) * K);
  const v4i rb = rsrc_words(w + (size_t)n0 * (size_t)K, (int64_t)(N - n0) * K);
  uint32_t off[C::kPerWave];
  int kc[C::kPerWave];
#pragma unroll
  for (int s = 0; s < C::kPerWave; ++s) {
    const bool isA = s < C::kPerWaveA;
    const int copy = isA ? wave * C::kPerWaveA + s : wave * C::kPerWaveB + (s - C::kPerWaveA);
    const int row = copy * C::kRowsPerCopy + lane / C::kChunks;
    const int chunk = (lane % C::kChunks) ^ C::swz(row);
    kc[s] = chunk * 16;
    const bool valid = isA ? (m0 + row < M) : (n0 + row < N);
    off[s] = valid ? (uint32_t)(row * K + chunk * 16) : kOutOfRange;
  }
  // Copies of a stage into `base`; part p >= 0 issues only the copies s
  // with s KS / kPerWave == p (one part per 32-k step of `compute`).
  auto issue = [&](int8_t* base, int stage, int part = -1) __attribute__((always_inline)) {
    const int k0 = stage * BK;
#pragma unroll
    for (int s = 0; s < C::kPerWave; ++s) {
      if (part >= 0 && s * (BK / 32) / C::kPerWave != part) continue;
      const bool isA = s < C::kPerWaveA;
      const int copy = isA ? wave * C::kPerWaveA + s : wave * C::kPerWaveB + (s - C::kPerWaveA);
      const uint32_t o = (k0 + kc[s] < kend) ? off[s] + (uint32_t)k0 : kOutOfRange;
      const int8_t* dst = base + (isA ? 0 : BM * BK) + copy * 1024;
      copy_to_lds(isA ? ra : rb, lds_addr(dst), o);
    }
  };

  v16i acc[C::kTM][C::kTN];
#pragma unroll
  for (int i = 0; i < C::kTM; ++i)
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) acc[i][j] = v16i{};

  // Fragment reads: row (l % 32) of each 32-row tile, logical chunk
  // 2 ks + l / 32, stored at chunk ^ swz(row) (tile bases are multiples of
  // 32 rows, so swz depends on the lane only).
  const int rl = lane & 31;
  const int sw = C::swz(rl);
  const int arow = (wm * C::kWTM + rl) * BK;
  const int brow = (BM + wn * C::kWTN + rl) * BK;
  constexpr int KS = BK / 32;

  auto compute = [&](const int8_t* buf, int8_t* nxt, int nstage) __attribute__((always_inline)) {
    v4i af[2][C::kTM], bf[2][C::kTN];
    auto read = [&](int ks, int slot) __attribute__((always_inline)) {
      const int c = ((2 * ks + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int i = 0; i < C::kTM; ++i) af[slot][i] = *reinterpret_cast<const v4i*>(buf + arow + i * 32 * BK + c);
#pragma unroll
      for (int j = 0; j < C::kTN; ++j) bf[slot][j] = *reinterpret_cast<const v4i*>(buf + brow + j * 32 * BK + c);
    };
    read(0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      issue(nxt, nstage, ks);
      if (ks + 1 < KS) read(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[ks & 1][i], bf[ks & 1][j], acc[i][j], 0, 0, 0);
    }
  };
  // One pipeline step: stage `stage` sits in `cur`; the copies of stage
  // stage + RING - 1 go into `nxt` (the buffer of stage - 1), a part before
  // each 32-k step's MFMAs rather than all before the first: a wave that
  // issued them all at once waited on their issue (MI355X, same bits, with
  // the weights in the memory-side cache: 512 x 9728 x 2560 23.0 -> 21.2 us,
  // 1024 x 5120 x 5120 38.6-40.9 -> 36.1-36.7 us; with the weights from HBM
  // 0-6%, e.g. 1024 x 5120 x 9728 66.4 -> 62.9 us, 36 shapes of M = 128 to
  // 1024 summing to 1148 against 1167 us).
  auto step = [&](const int8_t* cur, int8_t* nxt, int stage) __attribute__((always_inline)) {
    wait_vmcnt<(RING - 2) * C::kPerWave>();
    __syncthreads();
    compute(cur, nxt, stage + RING - 1);
  };

  // Stage count padded to a multiple of the ring: padded stages read zeros.
  const int nkr = (ke - kb + RING - 1) / RING * RING;
  issue(lds0, kb);
  if constexpr (RING > 2) issue(lds1, kb + 1);
  if constexpr (RING > 3) issue(lds2, kb + 2);
  for (int k = kb; k < kb + nkr; k += RING) {
    if constexpr (RING == 2) {
      step(lds0, lds1, k);
      step(lds1, lds0, k + 1);
    } else if constexpr (RING == 3) {
      step(lds0, lds2, k);
      step(lds1, lds0, k + 1);
      step(lds2, lds1, k + 2);
    } else {
      step(lds0, lds3, k);
      step(lds1, lds0, k + 1);
      step(lds2, lds1, k + 2);
      step(lds3, lds2, k + 3);
    }
  }
  wait_vmcnt<0>();  // no copy may land in LDS after the workgroup ends

  // Register r of tile (i, j) holds row mb + 32 i + (r / 4) * 8 + r % 4 and
  // column nb + 32 j; interior tiles store without per-element bounds checks.
  const int mb = m0 + wm * C::kWTM + (lane >> 5) * 4, nb = n0 + wn * C::kWTN + rl;
  const bool full = m0 + BM <= M && n0 + BN <= N;
  if (splits > 1) {
    int32_t* yi = reinterpret_cast<int32_t*>(y);
    auto partial = [&](auto checked) __attribute__((always_inline)) {
      constexpr bool CHK = decltype(checked)::value;
#pragma unroll
      for (int j = 0; j < C::kTN; ++j) {
        const int n = nb + j * 32;
        if (CHK && n >= N) continue;
#pragma unroll
        for (int i = 0; i < C::kTM; ++i) {
          const int mr = mb + i * 32;
          int32_t* p = yi + (size_t)mr * (size_t)N + (size_t)n;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int dr = (r >> 2) * 8 + (r & 3);
            if (CHK && mr + dr >= M) continue;
            __hip_atomic_fetch_add(p + (size_t)dr * (size_t)N, acc[i][j][r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    };
    if (full) partial(std::false_type{});
    else partial(std::true_type{});
    return;
  }

  // The tile's row and column scales, loaded once into LDS (as in
  // gemm_pp_kernel) instead of per element inside the store loop.  Every
  // wave has waited for its own copies above; the barrier orders these
  // writes after all of them and after every wave's last fragment read.
  __shared__ __attribute__((aligned(16))) float sa_l[BM];
  __shared__ float sw_l[BN];
  __syncthreads();
  for (int t = threadIdx.x; t < BM + BN; t += C::kNT) {
    if (t < BM) sa_l[t] = m0 + t < M ? s_a[m0 + t] : 0.0f;
    else sw_l[t - BM] = n0 + t - BM < N ? s_w[n0 + t - BM] : 0.0f;
  }
  __syncthreads();
  auto epilogue = [&](auto with_acc, auto checked) __attribute__((always_inline)) {
    constexpr bool ACC = decltype(with_acc)::value, CHK = decltype(checked)::value;
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) {
      const int mr = mb + i * 32;
      float sa[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4f v = *reinterpret_cast<const v4f*>(sa_l + (mr - m0) + 8 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) sa[4 * g + e] = v[e];
      }
#pragma unroll
      for (int j = 0; j < C::kTN; ++j) {
        const int n = nb + j * 32;
        if (CHK && n >= N) continue;
        const float swn = sw_l[n - n0];
        float* yp = y + (size_t)mr * (size_t)N + (size_t)n;
        int32_t* ap = ACC ? acc_out + (size_t)mr * (size_t)N + (size_t)n : nullptr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dr = (r >> 2) * 8 + (r & 3);
          if (CHK && mr + dr >= M) continue;
          const int a = acc[i][j][r];
          if constexpr (ACC) ap[(size_t)dr * (size_t)N] = a;
          const float t = (float)a * sa[r];
          yp[(size_t)dr * (size_t)N] = t * swn;
        }
      }
    }
  };
  if (acc_out) {
    if (full) epilogue(std::true_type{}, std::false_type{});
    else epilogue(std::true_type{}, std::true_type{});
  } else {
    if (full) epilogue(std::false_type{}, std::false_type{});
    else epilogue(std::false_type{}, std::true_type{});
  }
}

// Split-K helpers: zero y (as int32) before the partial tiles are added, and
// turn the exact int32 sums into the per-channel fp32 epilogue afterwards,
// in place, one element per thread.
__global__ __launch_bounds__(256) void zero_kernel(int32_t* __restrict__ p, int64_t n) {
  // One 16-byte chunk per thread; the last chunk may be partial.  p need only
  // be 4-byte aligned (the C ABI's rule for y): the 16-byte stores are then
  // dword aligned, which gfx950 global memory accesses allow.
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    *reinterpret_cast<v4i*>(p + i) = v4i{0, 0, 0, 0};
  } else {
    for (int64_t j = i; j < n; ++j) p[j] = 0;
  }
}

__global__ __launch_bounds__(256) void finalize_kernel(float* __restrict__ y, int32_t* __restrict__ acc_out,
                                                       const float* __restrict__ s_a, const float* __restrict__ s_w,
                                                       int M, int N) {
  // Four consecutive elements per thread (16-byte accesses, dword aligned at
  // least), which may run across the end of a row.
  const int64_t total = (int64_t)M * N;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= total) return;
  int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
  const int cnt = total - i < 4 ? (int)(total - i) : 4;
  int a[4] = {0, 0, 0, 0};
  float o[4];
  if (cnt == 4) {
    const v4i v = *reinterpret_cast<const v4i*>(reinterpret_cast<const int32_t*>(y) + i);
    a[0] = v[0]; a[1] = v[1]; a[2] = v[2]; a[3] = v[3];
  } else {
    for (int e = 0; e < cnt; ++e) a[e] = reinterpret_cast<const int32_t*>(y)[i + e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float t = (float)a[e] * s_a[m];
    o[e] = t * s_w[n];
    if (++n == N) { n = 0; if (m + 1 < M) ++m; }
  }
  if (cnt == 4) {
    if (acc_out) *reinterpret_cast<v4i*>(acc_out + i) = v4i{a[0], a[1], a[2], a[3]};
    *reinterpret_cast<v4f*>(y + i) = v4f{o[0], o[1], o[2], o[3]};
  } else {
    for (int e = 0; e < cnt; ++e) {
      if (acc_out) acc_out[i + e] = a[e];
      y[i + e] = o[e];
    }
  }
}

// The same epilogue when N % 4 == 0 (every row then starts at a multiple of
// 16 bytes from y; y, acc and s_w need only be 4-byte aligned):
// one workgroup per 1024 columns of one row, so the row index and its scale
// are uniform over the workgroup and the column scales are one 16-byte load.
// (At M = 512, N = 2560 on MI355X: 3.5 us against 5.0 for the flat form.)
__global__ __launch_bounds__(256) void finalize_rows_kernel(float* __restrict__ y, int32_t* __restrict__ acc_out,
                                                            const float* __restrict__ s_a,
                                                            const float* __restrict__ s_w, int N, int pieces) {
  const int m = blockIdx.x / pieces;
  const int n = (blockIdx.x - m * pieces) * 1024 + 4 * threadIdx.x;
  if (n >= N) return;  // N % 4 == 0, so n + 4 <= N
  const size_t i = (size_t)m * (size_t)N + (size_t)n;
  const float sa = s_a[m];
  const v4i a = *reinterpret_cast<const v4i*>(reinterpret_cast<const int32_t*>(y) + i);
  const v4f sw = *reinterpret_cast<const v4f*>(s_w + n);
  v4f o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float t = (float)a[e] * sa;
    o[e] = t * sw[e];
  }
  if (acc_out) *reinterpret_cast<v4i*>(acc_out + i) = a;
  *reinterpret_cast<v4f*>(y + i) = o;
}

// Runs the in-place epilogue of a K-split launch on the int32 sums in y.
inline void launch_finalize(float* y, int32_t* acc, const float* s_a, const float* s_w, int M, int N,
                            hipStream_t st) {
  const int64_t pieces = (N + 1023) / 1024;
  if (N % 4 == 0 && (int64_t)M * pieces <= INT32_MAX) {
    finalize_rows_kernel<<<(unsigned)(M * pieces), 256, 0, st>>>(y, acc, s_a, s_w, N, (int)pieces);
  } else {
    const int64_t total = (int64_t)M * N;
    finalize_kernel<<<(unsigned)((total + 1023) / 1024), 256, 0, st>>>(y, acc, s_a, s_w, M, N);
  }
}

template <int BM, int BN, int BK, int WM, int WN, int RING, int OCC>
void launch(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc, int M,
            int N, int K, hipStream_t st, int splits = 1) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t total = (int64_t)M * N;
  if (splits > 1)
    zero_kernel<<<(unsigned)((total + 1023) / 1024), 256, 0, st>>>(reinterpret_cast<int32_t*>(y), total);
  gemm_dma_kernel<BM, BN, BK, WM, WN, RING, OCC><<<(unsigned)(tiles_m * tiles_n * splits), 64 * WM * WN, 0, st>>>(
      q, s_a, w, s_w, y, acc, M, N, K, tiles_m, tiles_n, splits);
  if (splits > 1) launch_finalize(y, acc, s_a, s_w, M, N, st);
}

// Block-scale W8A8 on the direct-to-LDS pipeline.  Each stage also carries
// the fp16 block scales of its BK / 32 blocks for the tile's BN columns: a
// 2-byte copy writes lane i's value zero-extended into the dword at LDS base
// + 4 i, so one wave-wide copy moves one block's scales for 64 columns, and
// block ks of column c sits at dword ks * BN + c of the stage's scale area.
// Per 32-k block, each 32x32 tile is one MFMA started from zero; its exact
// int32 result is folded into fp32 accumulators in ascending block order:
// f = fmaf((float)P_b, (float)d[n][b], f); at the end y = f * s_a[m].
template <int BM, int BN, int WM, int WN, int RING, int OCC, bool PARTIALS>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_block_kernel(const int8_t* __restrict__ q,
                                                                       const float* __restrict__ s_a,
                                                                       const int8_t* __restrict__ w,
                                                                       const uint16_t* __restrict__ d,
                                                                       float* __restrict__ y,
                                                                       int32_t* __restrict__ partials, int M, int N,
                                                                       int K, int tiles_m, int tiles_n) {
  constexpr int BK = 128;
  constexpr int KS = BK / 32;  // blocks per stage
  using C = Cfg<BM, BN, BK, WM, WN, RING>;
  constexpr int kDCopies = KS * BN / 64;
  constexpr int kPerWaveD = kDCopies / C::kNW;
  static_assert(kDCopies % C::kNW == 0, "scale copies must divide among waves");
  constexpr int kPerWave = C::kPerWave + kPerWaveD;
  constexpr int kDOff = (BM + BN) * BK;          // scale area within a stage
  constexpr int kStage = kDOff + KS * BN * 4;
  static_assert(RING * kStage <= 160 * 1024, "LDS ring exceeds 160 KiB");
  static_assert((RING - 2) * kPerWave < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) int8_t lds0[kStage];
  __shared__ __attribute__((aligned(1024))) int8_t lds1[kStage];
  __shared__ __attribute__((aligned(1024))) int8_t lds2[RING > 2 ? kStage : 16];
  __shared__ __attribute__((aligned(1024))) int8_t lds3[RING > 3 ? kStage : 16];

  int tm, tn;
  tile_of(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  // The wave index through readfirstlane: the copies' LDS destinations are
  // then scalar (no readfirstlane per copy).
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / WN, wn = wave % WN;
  const int NB = K / 32;

  const v4i ra = rsrc_words(q + (size_t)m0 * (size_t)K, (int64_t)(M - m0) * K);
  const v4i rb = rsrc_words(w + (size_t)n0 * (size_t)K, (int64_t)(N - n0) * K);
  const v4i rd = rsrc_words(d + (size_t)n0 * (size_t)NB, (int64_t)(N - n0) * NB * 2);
  uint32_t off[C::kPerWave];
#pragma unroll
  for (int s = 0; s < C::kPerWave; ++s) {
    const bool isA = s < C::kPerWaveA;
    const int copy = isA ? wave * C::kPerWaveA + s : wave * C::kPerWaveB + (s - C::kPerWaveA);
    const int row = copy * C::kRowsPerCopy + lane / C::kChunks;
    const int chunk = (lane % C::kChunks) ^ C::swz(row);
    const bool valid = isA ? (m0 + row < M) : (n0 + row < N);
    off[s] = valid ? (uint32_t)(row * K + chunk * 16) : kOutOfRange;
  }
  // Scale copies of this wave: copy c holds block c / (BN / 64) of columns
  // (c % (BN / 64)) * 64 + lane.
  uint32_t doff[kPerWaveD > 0 ? kPerWaveD : 1];
  int dks[kPerWaveD > 0 ? kPerWaveD : 1];
#pragma unroll
  for (int s = 0; s < kPerWaveD; ++s) {
    const int c = wave * kPerWaveD + s;
    const int col = (c % (BN / 64)) * 64 + lane;
    dks[s] = c / (BN / 64);
    doff[s] = (n0 + col < N) ? (uint32_t)(col * NB * 2) : kOutOfRange;
  }
  // Copies of a stage into `base`; part p >= 0 issues only the copies s
  // (operands, then scales) with s KS / kPerWave == p.
  auto issue = [&](int8_t* base, int stage, int part = -1) __attribute__((always_inline)) {
    const int k0 = stage * BK;
#pragma unroll
    for (int s = 0; s < C::kPerWave; ++s) {
      if (part >= 0 && s * KS / kPerWave != part) continue;
      const bool isA = s < C::kPerWaveA;
      const int copy = isA ? wave * C::kPerWaveA + s : wave * C::kPerWaveB + (s - C::kPerWaveA);
      // No per-lane check against K: bytes past K (the next row, or zeros past
      // the end of the buffer) only enter blocks past K, whose scales load as
      // zero, and fmaf(P, 0, f) leaves f unchanged.
      const uint32_t o = off[s] + (uint32_t)k0;
      const int8_t* dst = base + (isA ? 0 : BM * BK) + copy * 1024;
      copy_to_lds(isA ? ra : rb, lds_addr(dst), o);
    }
#pragma unroll
    for (int s = 0; s < kPerWaveD; ++s) {
      if (part >= 0 && (C::kPerWave + s) * KS / kPerWave != part) continue;
      const int b = stage * KS + dks[s];
      const uint32_t o = (b < NB) ? doff[s] + (uint32_t)(b * 2) : kOutOfRange;
      const int8_t* dst = base + kDOff + (wave * kPerWaveD + s) * 256;
      copy2_to_lds(rd, lds_addr(dst), o);
    }
  };

  float f[C::kTM][C::kTN][16];
#pragma unroll
  for (int i = 0; i < C::kTM; ++i)
#pragma unroll
    for (int j = 0; j < C::kTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) f[i][j][r] = 0.0f;

  const int rl = lane & 31;
  const int sw = C::swz(rl);
  const int arow = (wm * C::kWTM + rl) * BK;
  const int brow = (BM + wn * C::kWTN + rl) * BK;
  int ncol[C::kTN];
#pragma unroll
  for (int j = 0; j < C::kTN; ++j) ncol[j] = wn * C::kWTN + j * 32 + rl;

  // The eight-wave 128 x 128 instance issues the next stage's copies a part
  // before each block instead of all before the first (MI355X, M = 2048,
  // 17408 x 5120: 430-459 -> 415-424 us, same bits); the four-wave 128 x 64
  // and 64 x 64 instances were slower that way (M = 512: 124 -> 132 us).
  constexpr bool kSpread = C::kNW == 8;
  auto compute = [&](const int8_t* buf, int stage, int8_t* nxt) __attribute__((always_inline)) {
    const v16i zero = v16i{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (kSpread) issue(nxt, stage + RING - 1, ks);
      // Blocks past K (padding of the last stage and of the ring) read zero
      // operands and zero scales: fmaf(0, 0, f) returns f unchanged (f starts
      // at +0 and can never become -0), so they need no branch.
      const int b = stage * KS + ks;
      const int c = ((2 * ks + (lane >> 5)) ^ sw) * 16;
      v4i af[C::kTM], bf[C::kTN];
      float dv[C::kTN];
#pragma unroll
      for (int i = 0; i < C::kTM; ++i) af[i] = *reinterpret_cast<const v4i*>(buf + arow + i * 32 * BK + c);
#pragma unroll
      for (int j = 0; j < C::kTN; ++j) {
        bf[j] = *reinterpret_cast<const v4i*>(buf + brow + j * 32 * BK + c);
        const uint32_t hbits = *reinterpret_cast<const uint32_t*>(buf + kDOff + (ks * BN + ncol[j]) * 4);
        dv[j] = half_bits_to_float((uint16_t)hbits);
        // fp32 from here on: folded into the fma as a binary16 operand, the
        // compiler emits v_fma_mix_f32, which issues slower than v_fmac_f32
        // (M = 2048, 17408 x 5120: 505 -> 470 us).
        asm volatile("" : "+v"(dv[j]));
      }
      // All MFMAs of the block first, then the folds at a raised wave
      // priority: the workgroups sharing a SIMD then tend to alternate, one
      // folding on the VALU while the other's MFMAs run.
      v16i p[C::kTM][C::kTN];
#pragma unroll
      for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) p[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], zero, 0, 0, 0);
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) {
#pragma unroll
          for (int r = 0; r < 16; ++r) f[i][j][r] = __builtin_fmaf((float)p[i][j][r], dv[j], f[i][j][r]);
          if constexpr (PARTIALS) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int m = m0 + wm * C::kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
              const int n = n0 + ncol[j];
              if (m < M && n < N && b < NB) partials[((size_t)m * (size_t)N + (size_t)n) * (size_t)NB + b] = p[i][j][r];
            }
          }
        }
      __builtin_amdgcn_s_setprio(0);
    }
  };
  auto step = [&](const int8_t* cur, int8_t* nxt, int stage) __attribute__((always_inline)) {
    wait_vmcnt<(RING - 2) * kPerWave>();
    __syncthreads();
    if constexpr (!kSpread) issue(nxt, stage + RING - 1);
    compute(cur, stage, nxt);
  };

  const int nk = (K + BK - 1) / BK;
  const int nkr = (nk + RING - 1) / RING * RING;
  issue(lds0, 0);
  if constexpr (RING > 2) issue(lds1, 1);
  if constexpr (RING > 3) issue(lds2, 2);
  for (int k = 0; k < nkr; k += RING) {
    if constexpr (RING == 2) {
      step(lds0, lds1, k);
      step(lds1, lds0, k + 1);
    } else if constexpr (RING == 3) {
      step(lds0, lds2, k);
      step(lds1, lds0, k + 1);
      step(lds2, lds1, k + 2);
    } else {
      step(lds0, lds3, k);
      step(lds1, lds0, k + 1);
      step(lds2, lds1, k + 2);
      step(lds3, lds2, k + 3);
    }
  }
  wait_vmcnt<0>();

#pragma unroll
  for (int j = 0; j < C::kTN; ++j) {
    const int n = n0 + ncol[j];
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * C::kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < M) y[(size_t)m * (size_t)N + (size_t)n] = f[i][j][r] * s_a[m];
      }
    }
  }
}

// The partial-sum output (a debugging aid) is a separate instantiation, so
// that the hot loop of the plain call carries no per-block stores.
template <int BM, int BN, int WM, int WN, int RING, int OCC, bool WITH_PARTIALS = true>
void launch_block(const int8_t* q, const float* s_a, const int8_t* w, const uint16_t* d, float* y, int32_t* partials,
                  int M, int N, int K, hipStream_t st) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  // The variant that also stores every block partial keeps more values live
  // (the partial tiles and their addresses); it is built for one workgroup
  // per CU so that it has the register file to itself and does not spill.
  // WITH_PARTIALS = false: that variant is not built (partials must be null).
  if constexpr (WITH_PARTIALS) {
    if (partials) {
      gemm_block_kernel<BM, BN, WM, WN, RING, 1, true><<<(unsigned)(tiles_m * tiles_n), 64 * WM * WN, 0, st>>>(
          q, s_a, w, d, y, partials, M, N, K, tiles_m, tiles_n);
      return;
    }
  }
  gemm_block_kernel<BM, BN, WM, WN, RING, OCC, false><<<(unsigned)(tiles_m * tiles_n), 64 * WM * WN, 0, st>>>(
      q, s_a, w, d, y, nullptr, M, N, K, tiles_m, tiles_n);
}

// Q4_K-native W4A8 on the repacked planes: packed 4-bit codes w4 [N][K/2]
// (32 bytes per pair of 32-k sub-blocks: byte l holds k = l in its low nibble
// and k = 32 + l in its high one) and the 16-byte super-block headers hdr
// [N][K/256][16] (d, dmin, 6-bit scales and mins).  Per 32-k sub-block: P =
// sum code * a (exact int32 from an MFMA started at zero) and S = sum a (exact
// int32, v_dot4 over the activation tile in LDS, once per workgroup and
// stage), folded in ascending sub-block order: f = fmaf((float)P, D, f);
// f = fmaf(-(float)S, Mn, f); y = f * s_a[m], with D = d * sc and Mn = dmin *
// m decoded from the header (exact in fp32).
//
// Direct-to-LDS pipeline as in gemm_block_kernel, a stage of 128 k: A rows of
// 128 bytes, B rows of 64 packed bytes (chunk c of row r stored at c ^ ((r /
// 4) % 4), so 16 consecutive rows reading one chunk hit 16 distinct 16-byte
// bank groups), and the headers of the stage's super-block (one 16-byte copy
// per column).  After a stage has landed, the workgroup decodes its BN x 4
// (D, Mn) pairs and computes its BM x 4 values of -S into LDS (one barrier),
// then folds; the fragment reads unpack the codes with one shift and mask per
// dword.  (-S from an MFMA against ones, converted per lane in every wave,
// cost 16 converts per 32 rows and sub-block: M = 2048, 17408 x 5120, 650 ->
// 600 us without them.)
template <int BM, int BN, int WM, int WN, int RING, int OCC>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_q4k_kernel(const int8_t* __restrict__ q,
                                                                     const float* __restrict__ s_a,
                                                                     const uint8_t* __restrict__ w4,
                                                                     const uint8_t* __restrict__ hdr,
                                                                     float* __restrict__ y, int M, int N, int K,
                                                                     int tiles_m, int tiles_n) {
  constexpr int BK = 128;
  constexpr int KS = BK / 32;  // sub-blocks per stage
  using C = Cfg<BM, BN, BK, WM, WN, RING>;
  constexpr int NT = C::kNT;
  constexpr int kCopiesB = BN * (BK / 2) / 1024;  // packed B: 16 rows of 64 bytes per copy
  constexpr int kCopiesH = BN * 16 / 256;         // headers: 4-byte copies, 16 columns per copy
  static_assert(kCopiesB % C::kNW == 0 && kCopiesH % C::kNW == 0, "copies must divide among waves");
  constexpr int kPerWaveB = kCopiesB / C::kNW;
  constexpr int kPerWaveH = kCopiesH / C::kNW;
  constexpr int kBOff = BM * BK;                  // packed B within a stage
  constexpr int kHOff = kBOff + BN * (BK / 2);    // headers within a stage
  constexpr int kStage = kHOff + BN * 16;
  static_assert(RING * kStage + 2 * KS * BN * 4 + KS * BM * 4 <= 160 * 1024 / OCC, "LDS");
  static_assert(KS * BM % NT == 0, "-S values must divide among threads");
  __shared__ __attribute__((aligned(1024))) int8_t lds0[kStage];
  __shared__ __attribute__((aligned(1024))) int8_t lds1[kStage];
  __shared__ __attribute__((aligned(1024))) int8_t lds2[RING > 2 ? kStage : 16];
  __shared__ float dsc[KS][BN], msc[KS][BN];  // decoded D and Mn of the stage being folded
  __shared__ __attribute__((aligned(16))) float nsc[KS][BM];  // -S of the stage's sub-blocks, per activation row

  int tm, tn;
  tile_of(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // scalar
  const int wm = wave / WN, wn = wave % WN;
  const int NS = K / 256;

  const v4i ra = rsrc_words(q + (size_t)m0 * (size_t)K, (int64_t)(M - m0) * K);
  const v4i rb = rsrc_words(w4 + (size_t)n0 * (size_t)(K / 2), (int64_t)(N - n0) * (K / 2));
  const v4i rh = rsrc_words(hdr + (size_t)n0 * (size_t)NS * 16, (int64_t)(N - n0) * NS * 16);
  // A copies: as gemm_dma_kernel.  Rows past M or N read zeros (out of range).
  uint32_t offa[C::kPerWaveA];
#pragma unroll
  for (int s = 0; s < C::kPerWaveA; ++s) {
    const int copy = wave * C::kPerWaveA + s;
    const int row = copy * C::kRowsPerCopy + lane / C::kChunks;
    const int chunk = (lane % C::kChunks) ^ C::swz(row);
    offa[s] = (m0 + row < M) ? (uint32_t)(row * K + chunk * 16) : kOutOfRange;
  }
  // B copies: lane -> row copy * 16 + lane / 4, LDS slot lane % 4, which holds
  // logical chunk (lane % 4) ^ ((row / 4) % 4) of the row's 64 packed bytes.
  // K is a multiple of 256 (whole super-blocks), so a 128-k stage is either
  // inside K or past it as a whole.
  uint32_t offb[kPerWaveB];
#pragma unroll
  for (int s = 0; s < kPerWaveB; ++s) {
    const int copy = wave * kPerWaveB + s;
    const int row = copy * 16 + lane / 4;
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    offb[s] = (n0 + row < N) ? (uint32_t)(row * (K / 2) + chunk * 16) : kOutOfRange;
  }
  // Header copies, 4 bytes per lane: copy c moves dword lane % 4 of the
  // header of column 16 c + lane / 4, every wave the same number of copies
  // (a branch around an LDS copy, even a uniform one, made the compiler spill
  // hundreds of registers here).
  uint32_t offh[kPerWaveH];
#pragma unroll
  for (int s = 0; s < kPerWaveH; ++s) {
    const int col = (wave * kPerWaveH + s) * 16 + lane / 4;
    offh[s] = (n0 + col < N) ? (uint32_t)(col * NS * 16 + (lane & 3) * 4) : kOutOfRange;
  }
  // Copies of a stage into `base`; part p >= 0 issues only the copies s
  // (operands, packed codes, then headers) with s KS / kQ == p.
  auto issue = [&](int8_t* base, int stage, int part = -1) __attribute__((always_inline)) {
    constexpr int kQ = C::kPerWaveA + kPerWaveB + kPerWaveH;
    const int k0 = stage * BK;
    // The LDS address of the stage as a scalar once (not a pointer per copy,
    // which the compiler kept in VGPRs and read back with readfirstlane).
    const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(base));
#pragma unroll
    for (int s = 0; s < C::kPerWaveA; ++s) {
      // No check against K on the operand copies: a stage past K (ring
      // padding) meets zero headers below, so both fmas leave f unchanged.
      if (part >= 0 && s * KS / kQ != part) continue;
      const uint32_t o = offa[s] + (uint32_t)k0;
      copy_to_lds(ra, lb + (uint32_t)((wave * C::kPerWaveA + s) * 1024), o);
    }
#pragma unroll
    for (int s = 0; s < kPerWaveB; ++s) {
      if (part >= 0 && (C::kPerWaveA + s) * KS / kQ != part) continue;
      const uint32_t o = offb[s] + (uint32_t)(k0 / 2);
      copy_to_lds(rb, lb + (uint32_t)(kBOff + (wave * kPerWaveB + s) * 1024), o);
    }
#pragma unroll
    for (int s = 0; s < kPerWaveH; ++s) {
      if (part >= 0 && (C::kPerWaveA + kPerWaveB + s) * KS / kQ != part) continue;
      const uint32_t o = (k0 < K && offh[s] != kOutOfRange) ? offh[s] + (uint32_t)(stage / 2) * 16u : kOutOfRange;
      copy4_to_lds(rh, lb + (uint32_t)(kHOff + (wave * kPerWaveH + s) * 256), o);
    }
  };

  float f[C::kTM][C::kTN][16];
#pragma unroll
  for (int i = 0; i < C::kTM; ++i)
#pragma unroll
    for (int j = 0; j < C::kTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) f[i][j][r] = 0.0f;

  const int rl = lane & 31;
  const int sw = C::swz(rl);
  const int swb = (rl >> 2) & 3;
  const int arow = (wm * C::kWTM + rl) * BK;
  const int brow = kBOff + (wn * C::kWTN + rl) * (BK / 2);
  int ncol[C::kTN];
#pragma unroll
  for (int j = 0; j < C::kTN; ++j) ncol[j] = wn * C::kWTN + j * 32 + rl;

  // Decode the stage's (D, Mn) pairs: thread t takes column t % BN and
  // sub-blocks KS * (t / BN) / (NT / BN) onwards of the stage (the stage is
  // half of super-block stage / 2: sub-blocks 4 (stage % 2) + ks).
  auto decode = [&](const int8_t* buf, int stage) __attribute__((always_inline)) {
    constexpr int kPer = KS * BN / NT;  // pairs per thread
    const int col = threadIdx.x % BN, ks0 = (threadIdx.x / BN) * kPer;
    const v4i h = *reinterpret_cast<const v4i*>(buf + kHOff + col * 16);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      float D, Mn;
      q4k_scale_min(h, 4 * (stage & 1) + ks0 + e, D, Mn);
      dsc[ks0 + e][col] = D;
      msc[ks0 + e][col] = Mn;
    }
    // -S of every (sub-block, row) of the stage, from the activation tile in
    // LDS (chunk c of row r at (c ^ swz(r)) * 16): exact int32, then fp32.
#pragma unroll
    for (int e = 0; e < KS * BM / NT; ++e) {
      const int idx = (int)threadIdx.x + NT * e;
      const int ks = idx / BM, row = idx % BM;
      const int8_t* ar = buf + row * BK;
      const v4i x0 = *reinterpret_cast<const v4i*>(ar + ((2 * ks) ^ C::swz(row)) * 16);
      const v4i x1 = *reinterpret_cast<const v4i*>(ar + ((2 * ks + 1) ^ C::swz(row)) * 16);
      int t = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        t = __builtin_amdgcn_sdot4(x0[u], 0x01010101, t, false);
        t = __builtin_amdgcn_sdot4(x1[u], 0x01010101, t, false);
      }
      nsc[ks][row] = -(float)t;
    }
  };
  // As in the block-scale kernel, the eight-wave 128 x 128 instance issues
  // the next stage's copies a part before each sub-block (MI355X, M = 2048,
  // 17408 x 5120: 568-586 -> 551-563 us; M = 4096 1100 -> 1072-1082 us; same
  // bits); the four-wave 64 x 64 instance was slower that way (M = 64: 48.6
  // -> 52.8 us).
  constexpr bool kSpread = C::kNW == 8;
  auto compute = [&](const int8_t* buf, int8_t* nxt, int nstage) __attribute__((always_inline)) {
    const v16i zero = v16i{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (kSpread) issue(nxt, nstage, ks);
      // Sub-blocks past K read zero operands and zero scales: both fmas
      // return f unchanged (f starts at +0 and never becomes -0).
      const int c = ((2 * ks + (lane >> 5)) ^ sw) * 16;
      const int cb = ((2 * (ks >> 1) + (lane >> 5)) ^ swb) * 16;  // packed chunk of this lane's 16 k
      const int nib = (ks & 1) * 4;                               // odd sub-blocks: high nibbles
      v4i af[C::kTM], bf[C::kTN];
      float dv[C::kTN], mv[C::kTN];
#pragma unroll
      for (int i = 0; i < C::kTM; ++i) af[i] = *reinterpret_cast<const v4i*>(buf + arow + i * 32 * BK + c);
#pragma unroll
      for (int j = 0; j < C::kTN; ++j) {
        const v4i p = *reinterpret_cast<const v4i*>(buf + brow + j * 32 * (BK / 2) + cb);
#pragma unroll
        for (int e = 0; e < 4; ++e) bf[j][e] = (int)(((uint32_t)p[e] >> nib) & 0x0f0f0f0fu);
        dv[j] = dsc[ks][ncol[j]];
        mv[j] = msc[ks][ncol[j]];
      }
#pragma unroll
      for (int i = 0; i < C::kTM; ++i) {
        // -S of this lane's 16 rows (rows 8 (r / 4) + 4 (lane / 32) + r % 4 of the tile)
        float ns[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const v4f v = *reinterpret_cast<const v4f*>(&nsc[ks][wm * C::kWTM + i * 32 + 8 * g + 4 * (lane >> 5)]);
#pragma unroll
          for (int e = 0; e < 4; ++e) ns[4 * g + e] = v[e];
        }
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) {
          const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], zero, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            f[i][j][r] = __builtin_fmaf((float)p[r], dv[j], f[i][j][r]);
            f[i][j][r] = __builtin_fmaf(ns[r], mv[j], f[i][j][r]);
          }
        }
      }
      // keeps the next sub-block's fragment reads and unpacking after this
      // one's folds (hoisting them spills registers)
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Iteration: wait for this wave's copies of the stage, barrier (all copies
  // landed, every wave done with the previous stage and its decoded scales),
  // start the copies of stage + RING - 1, decode the scales, barrier, fold.
  auto step = [&](const int8_t* cur, int8_t* nxt, int stage) __attribute__((always_inline)) {
    wait_vmcnt<0>();
    __syncthreads();
    if constexpr (!kSpread) issue(nxt, stage + RING - 1);
    decode(cur, stage);
    __syncthreads();
    compute(cur, nxt, stage + RING - 1);
  };

  static_assert(RING == 2 || RING == 3, "ring depth");
  const int nk = (K + BK - 1) / BK;
  const int nkr = (nk + RING - 1) / RING * RING;
  issue(lds0, 0);
  if constexpr (RING > 2) issue(lds1, 1);
  for (int k = 0; k < nkr; k += RING) {
    if constexpr (RING == 2) {
      step(lds0, lds1, k);
      step(lds1, lds0, k + 1);
    } else {
      step(lds0, lds2, k);
      step(lds1, lds0, k + 1);
      step(lds2, lds1, k + 2);
    }
  }
  wait_vmcnt<0>();

#pragma unroll
  for (int j = 0; j < C::kTN; ++j) {
    const int n = n0 + ncol[j];
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * C::kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < M) y[(size_t)m * (size_t)N + (size_t)n] = f[i][j][r] * s_a[m];
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int RING, int OCC>
void launch_q4k(const int8_t* q, const float* s_a, const uint8_t* w4, const uint8_t* hdr, float* y, int M, int N,
                int K, hipStream_t st) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  gemm_q4k_kernel<BM, BN, WM, WN, RING, OCC><<<(unsigned)(tiles_m * tiles_n), 64 * WM * WN, 0, st>>>(
      q, s_a, w4, hdr, y, M, N, K, tiles_m, tiles_n);
}

}  // namespace dma

template <int BM, int BN, int BK, int WM, int WN, bool W4, int OCC>
void launch_tiled(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc,
                  int M, int N, int K, hipStream_t st, int splits = 1) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t total = (int64_t)M * N;
  if (splits > 1)
    dma::zero_kernel<<<(unsigned)((total + 1023) / 1024), 256, 0, st>>>(reinterpret_cast<int32_t*>(y), total);
  gemm_tiled_kernel<BM, BN, BK, WM, WN, W4, OCC><<<(unsigned)(tiles_m * tiles_n * splits), 64 * WM * WN, 0, st>>>(
      q, s_a, w, s_w, y, acc, M, N, K, tiles_m, tiles_n, splits);
  if (splits > 1) dma::launch_finalize(y, acc, s_a, s_w, M, N, st);
}

}  // namespace tiled
}  // namespace prism
