// Ping-pong schedule of the int8 tiled GEMM (output tiles of 256 rows by BN =
// 192, 256 or 320 columns, eight waves, direct-to-LDS copies as in
// gemm_dma_kernel), launched persistently: one workgroup per CU walks a list
// of tiles.
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
// issues its share of the global -> LDS copies of the next stage); in the
// next phase the roles swap.  Group 1 starts one barrier late, so the two
// waves of a SIMD alternate and the MFMA unit always has queued work.
//
// Stages are BK bytes of k for all rows of the tile (256 of A, BN of B) in a
// ring of two LDS buffers.  Both groups issue the copies of stage s + 1
// during stage s (int8: spread over its phases; 4-bit: in its first read
// phase), into the buffer of stage s - 1, which both groups finished reading
// before the barrier of stage s's first phase.  Before the
// barrier that precedes the first read of stage s + 1 every wave waits
// (s_waitcnt vmcnt) for its own copies of that stage.  LDS layout, swizzle
// and out-of-range zeros are those of gemm_dma_kernel.
//
// Persistent launch: the grid has one workgroup per CU (or one per tile when
// there are fewer tiles).  The tiles are split into one contiguous range per
// XCD, sized by the number of workgroups the XCD receives, and workgroup r of
// an XCD runs tiles r, r + g, r + 2 g, ... of its XCD's range (g workgroups
// on the XCD), so the tiles running together on an XCD are neighbours and
// share operand panels in its L2.  The last copy of a tile's main loop
// already fetches stage 0 of the workgroup's next tile, which therefore lands
// while the tile's epilogue runs.  On MI355X at M = 8192, N = K = 5120
// (256 x 320 tiles, two per CU) this took 215 us to 202 us against one
// workgroup per tile; 4096 x 9728 x 2560: 125 -> 112 us; 2048 x 17408 x 5120:
// 210 -> 198 us; M = 2048, N = K = 5120 (256 x 256 tiles): 71 -> 64 us.
// What remains is the overlap of the operand copies with the MFMAs: at M =
// 8192, N = K = 5120 (uniform int8 data) the kernel takes about 150 us with
// the copies left out and 123 us with the MFMAs left out, 185 us with both;
// with two stages in the ring a stage's copies have one stage of MFMA time
// to land.  The y writes of all CUs finishing their last tiles together add
// 15-30 us (measured with the stores left out).
#pragma once

#include <type_traits>

#include "gemm_tiled_kernels.h"

namespace prism {
namespace tiled {
namespace dma {

// Tile id -> tile coordinates: groups of kGroupCols tile columns,
// column-major inside a group, so that consecutive ids share a few weight
// panels and many activation panels.  Measured on MI355X at M = 8192,
// N = K = 5120: 261 us against 280 us for groups of 8 tile rows.
__device__ inline void tile_coords_cols(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int kGroupCols = 4;
  const int per_group = kGroupCols * tiles_m;
  const int grp = id / per_group;
  const int first = grp * kGroupCols;
  const int gn = min(tiles_n - first, kGroupCols);
  const int in = id - grp * per_group;
  tn = first + in % gn;
  tm = in / gn;
}

// Workgroup barrier that the compiler may not move memory accesses across.
__device__ inline void pp_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt lgkmcnt(0), no wait on vmcnt or expcnt (gfx9 encoding).
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// W4: w holds packed signed 4-bit weights [N][K/2] (low nibble = even k).
// Their bytes are copied to LDS as they are and unpacked at fragment read:
// each nibble moves to the top half of a byte, which as int8 is 16 w, so the
// MFMAs sum 16 acc exactly and the epilogue shifts it back.  A stage of
// 128 k holds only 64 packed bytes of a weight row, and 64-byte row pieces
// copy much slower than 128-byte ones, so B moves in pairs of stages (256 k,
// 128 bytes per row) through a ring of two pair buffers after the A ring:
// every stage copies one half of the pair after the one being read (the
// BN / 64 copies per wave of a pair split as evenly as they go: stage 0 of
// a pair copies the larger half), with a cursor of its own, and stages are
// padded to whole pairs of pairs so that each tile starts in pair buffer 0.
template <int BK, int BN = 256, int KSP = 2, bool W4 = false>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(const int8_t* __restrict__ q, const float* __restrict__ s_a,
                                                        const int8_t* __restrict__ w, const float* __restrict__ s_w,
                                                        float* __restrict__ y, int32_t* __restrict__ acc_out, int M,
                                                        int N, int K, int tiles_m, int tiles_n) {
  constexpr int BM = 256, RING = 2;
  using C = Cfg<BM, BN, BK, 4, 2, RING>;  // copies and LDS rows of A and B (W4: BK bytes of a pair's row)
  constexpr int kPerWaveA = C::kPerWaveA;
  constexpr int kPerWaveB = C::kPerWaveB;       // int8: per stage; W4: per pair
  constexpr int kPerWave = kPerWaveA + kPerWaveB;
  constexpr int kHalf0 = (kPerWaveB + 1) / 2;   // W4: copies per wave of the first half of a pair
  constexpr int kHalf1 = kPerWaveB / 2;
  constexpr int kStage = W4 ? BM * BK : (BM + BN) * BK;  // a stage of the ring (W4: A only)
  constexpr int kPair = BN * BK;                         // W4: a pair buffer
  constexpr int kLds = RING * kStage + (W4 ? 2 * kPair : 0);
  constexpr int P = BK / (32 * KSP);  // read/compute phase pairs per stage (KSP 32-k steps each)
  constexpr int TM = 2, TN = BN / 64;
  static_assert(C::kNW == 8 && C::kPerWaveA * 8 == C::kCopiesA && C::kPerWaveB * 8 == C::kCopiesB, "eight waves");
  static_assert(!W4 || BK == 128, "W4: 128-k stages");
  static_assert(kLds <= 160 * 1024, "LDS exceeds 160 KiB");
  __shared__ __attribute__((aligned(1024))) int8_t lds[kLds];
  __shared__ __attribute__((aligned(16))) float sa_l[BM];
  __shared__ float sw_l[BN];

  // This workgroup's tiles: t, t + g, ... below t_end.
  const int T = tiles_m * tiles_n;
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  const int xcd = b % 8;
  const int g = G / 8 + (xcd < G % 8 ? 1 : 0);          // workgroups on this XCD
  const int before = xcd * (G / 8) + min(xcd, G % 8);   // workgroups on lower XCDs
  const int t_end = (int)((int64_t)T * (before + g) / G);
  int t = (int)((int64_t)T * before / G) + b / 8;
  if (t >= t_end) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave >> 2, wm = wave & 3;
  const int nk = (K + BK - 1) / BK;
  const int nkr = W4 ? (nk + 3) / 4 * 4 : (nk + RING - 1) / RING * RING;  // padded stages read zeros

  const int KB = W4 ? K / 2 : K;  // bytes of a weight row
  // Index of this wave's i-th B copy (W4: the first half of a pair holds
  // copies 0 .. 8 kHalf0 - 1, the second half the rest).
  auto b_copy = [&](int i) __attribute__((always_inline)) {
    if (!W4) return wave * kPerWaveB + i;
    return i < kHalf0 ? wave * kHalf0 + i : 8 * kHalf0 + wave * kHalf1 + (i - kHalf0);
  };

  // The byte offset within the stage's k range of a lane's chunk (chunk * 16)
  // is recomputed at each issue from the lane and the copy index instead of
  // being kept per copy: a few VALU operations in a read phase, against one
  // register per copy.
  auto chunk_a = [&](int copy) __attribute__((always_inline)) {
    return (lane % C::kChunks) ^ C::swz(copy * C::kRowsPerCopy + lane / C::kChunks);
  };

  // Byte offset of this lane's chunk in each of its copies at k = 0, relative
  // to the tile's first row.  Rows past M or N lie beyond the tile's buffer
  // bound (below) and read zeros.
  uint32_t off[kPerWave];
#pragma unroll
  for (int s = 0; s < kPerWave; ++s) {
    if (s < kPerWaveA) {
      const int copy = wave * kPerWaveA + s;
      off[s] = (uint32_t)((copy * C::kRowsPerCopy + lane / C::kChunks) * K + chunk_a(copy) * 16);
    } else {
      const int copy = b_copy(s - kPerWaveA);
      off[s] = (uint32_t)((copy * C::kRowsPerCopy + lane / C::kChunks) * KB + chunk_a(copy) * 16);
    }
  }
  auto sources = [&](int tile, v4i& ra, v4i& rb, int& m0, int& n0) __attribute__((always_inline)) {
    int tm, tn;
    tile_coords_cols(tile, tiles_m, tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
    ra = rsrc_words(q + (size_t)m0 * (size_t)K, (int64_t)(M - m0) * K);
    rb = rsrc_words(w + (size_t)n0 * (size_t)KB, (int64_t)(N - n0) * KB);
  };

  // Copy cursor: the next stage to copy starts at byte ck of k in the tile
  // with sources (ca, cb).  After the last (padded) stage of a tile it moves
  // to stage 0 of the next tile, whose copies read zeros if there is none.
  int m0, n0, m0n = 0, n0n = 0;
  v4i ca, cb, ran = v4i{0, 0, 0, 0}, rbn = v4i{0, 0, 0, 0};
  sources(t, ca, cb, m0, n0);
  int ck = 0;
  bool clive = true, has_next = false;
  // W4 pair cursor: the next pair to copy starts at packed byte bk of the
  // rows of source wb; after a tile's last pair it moves to pair 0 of the
  // next tile.  Half h of a pair is copied by the stage whose index within
  // its own pair is h, so the half is known where the copy is issued.
  v4i wb = cb;
  int bk = 0;
  bool blive = true;
  auto issue_half_pair = [&](int h) __attribute__((always_inline)) {
    const int s0 = kPerWaveA + (h == 0 ? 0 : kHalf0), s1 = h == 0 ? kPerWaveA + kHalf0 : kPerWave;
#pragma unroll
    for (int s = s0; s < s1; ++s) {
      const int copy = b_copy(s - kPerWaveA);
      const uint32_t o = (blive && bk + chunk_a(copy) * 16 < KB) ? off[s] + (uint32_t)bk : kOutOfRange;
      const int8_t* dst = lds + RING * kStage + ((bk / BK) & 1) * kPair + copy * 1024;
      copy_to_lds(wb, lds_addr(dst), o);
    }
    if (h == 1) {
      bk += BK;
      if (bk >= nkr / 2 * BK) {
        wb = rbn;
        bk = 0;
        blive = has_next;
      }
    }
  };
  // Copies of the next stage into ring buffer buf (W4: and half h of the
  // next pair), in kParts parts: int8 spreads a wave's copies over the read
  // and compute phases of the stage's first P - 1 phase pairs (copy s in part
  // s kParts / kNCopies; none in the last pair, which ends in the wait for
  // them) instead of issuing them all in the stage's first read phase.  The
  // copies of a stage take about as long as its MFMAs, and a wave that issued
  // all of them at once waited on their issue in that phase.  MI355X, same
  // bits: M = 8192, N = K = 5120 194-196 -> 183-185 us; 4096 x 9728 x 2560
  // 109-112 -> 104 us; 2048 x 5120 x 5120 (256 x 192, two phase pairs per
  // stage) 57 -> 54 us.  The 4-bit form (A copies and one half pair per
  // stage) was not faster spread (2048 x 12288 x 4096: 102-105 against
  // 102-103 us; 4096 x 12288 x 4096: 187 against 189-191 us).
  constexpr int kParts = W4 ? 1 : (P > 1 ? 2 * P - 2 : 1);
  constexpr int kNCopies = W4 ? kPerWaveA : kPerWave;
  auto issue_part = [&](int buf, int h, int part) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kNCopies; ++s) {
      if (s * kParts / kNCopies != part) continue;
      const bool isA = s < kPerWaveA;
      const int copy = isA ? wave * kPerWaveA + s : b_copy(s - kPerWaveA);
      const uint32_t o = (clive && ck + chunk_a(copy) * 16 < K) ? off[s] + (uint32_t)ck : kOutOfRange;
      const int8_t* dst = lds + buf * kStage + (isA ? 0 : BM * BK) + copy * 1024;
      copy_to_lds(isA ? ca : cb, lds_addr(dst), o);
    }
    if (part != kParts - 1) return;
    if constexpr (W4) issue_half_pair(h);
    ck += BK;
    if (ck >= nkr * BK) {
      ca = ran;
      cb = rbn;
      ck = 0;
      clive = has_next;
    }
  };
  auto issue = [&](int buf, int h) __attribute__((always_inline)) {
#pragma unroll
    for (int pt = 0; pt < kParts; ++pt) issue_part(buf, h, pt);
  };

  v16i acc[TM][TN];
  const int rl = lane & 31;
  const int sw = C::swz(rl);
  const int arow = (wm * 64 + rl) * BK;
  const int brow = W4 ? RING * kStage + (grp * (BN / 2) + rl) * BK : (BM + grp * (BN / 2) + rl) * BK;
  v4i af[TM][KSP], bf[TN][KSP];
  // Fragments of the (32 KSP)-k slice `half` of the stage in buffer `buf`:
  // logical chunk 2 (KSP half + ks) + lane / 32 of row (lane % 32) of each
  // 32-row tile, i.e. k = 32 (KSP half + ks) + 16 (lane / 32) + [0, 16).
  // Packed B (stage `buf` of the pair in pair buffer `pb`): the same 16 k are
  // the 8 bytes at 8 (lane / 32) of logical chunk 4 buf + KSP half + ks of
  // the pair's 128-byte row.
  auto read = [&](int buf, int half, int pb) __attribute__((always_inline)) {
    const int8_t* base = lds + buf * kStage;
    if constexpr (W4 && KSP == 2) {
      // Packed B with two 32-k steps per phase: lane half h takes k = 64 half
      // + 32 h + [0, 32) of the stage, one whole 16-byte chunk of the pair
      // row, and its A fragments the same k: chunks 4 half + 2 h and 4 half
      // + 2 h + 1.  One conflict-free 16-byte read per column tile and phase
      // instead of two 8-byte reads, whose lanes r and r + 16 hit the same
      // LDS banks (MI355X, 2048 x 12288 x 4096: 125-129 -> 120 us).
      // Step 0 then takes the 16 even k of those 32 and step 1 the 16 odd k
      // (any k order shared by A and B gives the same exact int32 sums): B's
      // fragments are the low nibbles moved up and the high nibbles in
      // place, two and one operations per dword, with no byte interleave;
      // A's 32 bytes are split into even and odd bytes once per 32-row tile
      // (8 byte permutes), where interleaving the nibbles took 20 operations
      // per column tile (MI355X: 2048 x 12288 x 4096 110 -> 104-108 us,
      // 4096 x 12288 x 4096 204-213 -> 197-198 us).
      const int8_t* pbase = lds + pb * kPair;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = ((4 * half + 2 * (lane >> 5) + ks) ^ sw) * 16;
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i][ks] = *reinterpret_cast<const v4i*>(base + arow + i * 32 * BK + c);
      }
      const int cb = ((4 * buf + 2 * half + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4i u = *reinterpret_cast<const v4i*>(pbase + brow + j * 32 * BK + cb);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          bf[j][0][d] = (int)(((uint32_t)u[d] << 4) & 0xF0F0F0F0u);  // even k: 16 w of the low nibbles
          bf[j][1][d] = (int)((uint32_t)u[d] & 0xF0F0F0F0u);         // odd k: 16 w of the high nibbles
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const v4i a0 = af[i][0], a1 = af[i][1];  // k 0..15 and 16..31 of the lane's 32
        v4i ev, od;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          ev[d] = (int)__builtin_amdgcn_perm((uint32_t)a0[2 * d + 1], (uint32_t)a0[2 * d], 0x06040200u);
          od[d] = (int)__builtin_amdgcn_perm((uint32_t)a0[2 * d + 1], (uint32_t)a0[2 * d], 0x07050301u);
          ev[d + 2] = (int)__builtin_amdgcn_perm((uint32_t)a1[2 * d + 1], (uint32_t)a1[2 * d], 0x06040200u);
          od[d + 2] = (int)__builtin_amdgcn_perm((uint32_t)a1[2 * d + 1], (uint32_t)a1[2 * d], 0x07050301u);
        }
        af[i][0] = ev;
        af[i][1] = od;
      }
      return;
    }
#pragma unroll
    for (int ks = 0; ks < KSP; ++ks) {
      const int c = ((2 * (KSP * half + ks) + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i][ks] = *reinterpret_cast<const v4i*>(base + arow + i * 32 * BK + c);
      if constexpr (W4) {
        const int cb4 = ((4 * buf + KSP * half + ks) ^ sw) * 16 + (lane >> 5) * 8;
        const int8_t* pbase = lds + pb * kPair;
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bf[j][ks] = unpack_w4_8(*reinterpret_cast<const v2i*>(pbase + brow + j * 32 * BK + cb4));
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j][ks] = *reinterpret_cast<const v4i*>(base + brow + j * 32 * BK + c);
      }
    }
  };
  // Consecutive MFMAs share their B fragment (column tile outer, row tile
  // inner): with uniform random int8 operands, where the matrix cores run
  // into the power limit, M = 8192, N = K = 5120 took 242-247 us in the
  // other order and 218-227 us in this one (the same bits; the stress
  // activations of the benchmark step are unaffected).
  auto mma = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KSP; ++ks)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i][ks], bf[j][ks], acc[i][j], 0, 0, 0);
  };

  if constexpr (W4) issue_half_pair(0);  // half 0 of the first tile's pair 0
  issue(0, 1);                           // stage 0 of the first tile (W4: and half 1 of pair 0)
  while (true) {
    const int t_next = t + g;
    has_next = t_next < t_end;
    if (has_next) sources(t_next, ran, rbn, m0n, n0n);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};
    wait_vmcnt<0>();
    pp_barrier();
    if (grp == 1) pp_barrier();  // group 1 runs one phase behind group 0
    __builtin_amdgcn_sched_barrier(0);

    for (int u = 0; u < nkr; u += RING) {
#pragma unroll
      for (int r = 0; r < RING; ++r) {
#pragma unroll
        for (int h = 0; h < P; ++h) {
          // read phase of slice h of stage u + r (buffer r)
          // Fragment reads first, then this phase's copies: their issue
          // overlaps the reads' latency (MI355X: 1-2%, e.g. M = 8192, N = K =
          // 5120 185-188 -> 182-184 us).
          read(r, h, (u >> 1) & 1);
          if (2 * h < kParts) issue_part((r + RING - 1) % RING, r, 2 * h);
          wait_lgkm0();
          if (h == P - 1 && grp == 1) wait_vmcnt<0>();
          __builtin_amdgcn_sched_barrier(0);
          pp_barrier();
          __builtin_amdgcn_sched_barrier(0);
          // compute phase.  int8 tiles with two 32-k steps per phase (256 x
          // 192 and 256 x 256) raise the wave's priority while it issues its
          // MFMAs, so the other group's reads and copies on the same SIMD do
          // not delay them (MI355X, same bits: 2048 x 5120 x 5120 69-75 ->
          // 63-72 us, 3072 x 5120 x 5120 84-85 -> 82 us; other shapes
          // within 1%).  The 320-wide tiles and the 4-bit ones were slower
          // that way.
          if constexpr (KSP == 2 && !W4) __builtin_amdgcn_s_setprio(1);
          mma();
          if constexpr (KSP == 2 && !W4) __builtin_amdgcn_s_setprio(0);
          if (2 * h + 1 < kParts) issue_part((r + RING - 1) % RING, r, 2 * h + 1);
          if (h == P - 1 && grp == 0) wait_vmcnt<0>();
          __builtin_amdgcn_sched_barrier(0);
          pp_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (grp == 0) pp_barrier();  // matches group 1's extra barrier at the start

    // Epilogue.  The tile's row and column scales are loaded once into LDS:
    // reading them per element from global memory inside the store loop (32
    // row scales per lane) cost about 44 of 270 us at M = 8192, N = K = 5120.
    // The previous tile's epilogue finished reading them before the first
    // barrier of this tile's main loop.  y is written with nontemporal stores
    // (it is not read again here; 1-3% faster on the shapes above).
    for (int i = threadIdx.x; i < BM + BN; i += 512) {
      if (i < BM) sa_l[i] = m0 + i < M ? s_a[m0 + i] : 0.0f;
      else sw_l[i - BM] = n0 + i - BM < N ? s_w[n0 + i - BM] : 0.0f;
    }
    __syncthreads();
    // Register r of tile (i, j) holds row mr + (r / 4) * 8 + r % 4, mr = mb +
    // 32 i + 4 (lane / 32), column nb + 32 j + lane % 32.  Interior tiles
    // (every tile of most shapes) store without per-element bounds checks.
    const int mb = m0 + wm * 64 + (lane >> 5) * 4, nb = n0 + grp * (BN / 2);
    const bool full = m0 + BM <= M && n0 + BN <= N;
    auto epilogue = [&](auto with_acc, auto checked) __attribute__((always_inline)) {
      constexpr bool ACC = decltype(with_acc)::value, CHK = decltype(checked)::value;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int mr = mb + i * 32;
        float sa[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const v4f v = *reinterpret_cast<const v4f*>(sa_l + (mr - m0) + 8 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) sa[4 * g + e] = v[e];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = nb + j * 32 + rl;
          if (CHK && n >= N) continue;
          const float swn = sw_l[n - n0];
          float* yp = y + (size_t)mr * (size_t)N + (size_t)n;
          int32_t* ap = ACC ? acc_out + (size_t)mr * (size_t)N + (size_t)n : nullptr;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int dr = (r >> 2) * 8 + (r & 3);
            if (CHK && mr + dr >= M) continue;
            const int a = W4 ? acc[i][j][r] >> 4 : acc[i][j][r];  // exact: 16 w sums to a multiple of 16
            if constexpr (ACC) __builtin_nontemporal_store(a, ap + (size_t)dr * (size_t)N);
            const float tv = (float)a * sa[r];
            __builtin_nontemporal_store(tv * swn, yp + (size_t)dr * (size_t)N);
          }
        }
      }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (acc_out) {
      if (full) epilogue(T_{}, F_{});
      else epilogue(T_{}, T_{});
    } else {
      if (full) epilogue(F_{}, F_{});
      else epilogue(F_{}, T_{});
    }
    if (!has_next) break;
    t = t_next;
    m0 = m0n;
    n0 = n0n;
  }
  wait_vmcnt<0>();  // no copy may land in LDS after the workgroup ends
}

// Number of compute units of the current device (cached per device).
int device_cus();

template <int BK, int BN = 256, int KSP = 2, bool W4 = false>
void launch_pp(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc, int M,
               int N, int K, hipStream_t st) {
  const int tiles_m = (M + 255) / 256, tiles_n = (N + BN - 1) / BN;
  const int64_t T = (int64_t)tiles_m * tiles_n;
  const int cus = device_cus();
  const unsigned grid = (unsigned)(T < cus ? T : cus);
  gemm_pp_kernel<BK, BN, KSP, W4><<<grid, 512, 0, st>>>(q, s_a, w, s_w, y, acc, M, N, K, tiles_m, tiles_n);
}

}  // namespace dma
}  // namespace tiled
}  // namespace prism
