// Small-M GEMM (M <= 64): W8A8 and W4A8 with per-channel scales.
//
// Exact int32 sums (StartLux-Prism README, "Why StartLux-Prism" and "How it
// works") make a split of K free: integer addition is associative, so any
// grouping of the k-range gives the same accumulator.  At small M the weights
// dominate the bytes, so this kernel is built to stream them from HBM:
//
//  * one workgroup owns 16 * CB output columns and all M rows; its WAVES
//    waves split K into contiguous ranges of 128-k units and reduce their
//    int32 partials in LDS;
//  * each wave issues all loads of a batch of U units at once (weights for
//    its CB column blocks and activation fragments for its MB row blocks)
//    before any MFMA, as branch-free buffer loads that read zeros outside the
//    matrices, so the weight stream is in flight from the first cycles;
//  * weights go from HBM straight into MFMA operand registers (no LDS: each
//    weight byte is used by one wave only); an activation fragment is used by
//    CB column blocks;
//  * v_mfma_i32_16x16x64_i8: lane l holds column (l % 16) of the weights and
//    row (l % 16) of the activations, k-group g = l / 16.  Both operands use
//    the same lane -> k assignment, so the integer sum is the plain dot
//    product whatever that assignment is.  In unit u, group g covers
//    k = 128 u + 32 g + [0, 16) in the first MFMA and + [16, 32) in the second;
//  * 4-bit weights are unpacked in registers: each nibble is moved to the top
//    half of a byte, which as int8 equals 16 * w, so the MFMA sums 16 * acc
//    exactly (|16 * acc| < 2^31 for K <= 131040) and an arithmetic shift by 4
//    recovers acc;
//  * epilogue per element, in a fixed order: y = ((float)acc * s_a[m]) * s_w[n].
#include "prism_internal.h"
#include "quant_math.h"
#include "../../include/prism.h"

namespace prism {
namespace {

constexpr int kUnitK = 128;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < (int64_t)kOutOfRange - 1 ? bytes : (int64_t)kOutOfRange - 1;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

__device__ inline v4i bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

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

// The body of the small-M GEMM, shared by gemm_small_kernel and the fused
// quantize + GEMM kernel below.
// EARLY: before() is called first, then the first batch of weights is
// requested, then wait() is called, after which q (codes, rows a_stride
// bytes apart) and s_a are read from LDS.
struct NoWait {
  __device__ void operator()() const {}
};

template <int MB, int CB, bool W4, int WAVES, int U, bool EARLY = false, class Before = NoWait,
          class Wait = NoWait>
__device__ inline void small_gemm(const int8_t* q, const float* s_a, const int8_t* __restrict__ w,
                                  const float* __restrict__ s_w, float* __restrict__ y,
                                  int32_t* __restrict__ acc_out, int M, int N, int K, int G,
                                  Before before = Before(), Wait wait = Wait(), int a_stride = 0) {
  __shared__ int red[WAVES][CB * MB * 4][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  // Columns [n0, n1) of this workgroup: blocks of 16 CB (G == 0), or the
  // b-th of G even shares of N (G > 0; the host makes every share fit in
  // 16 CB columns), so that every CU streams the same number of weight rows.
  const int n0 = G > 0 ? (int)((int64_t)blockIdx.x * N / G) : blockIdx.x * 16 * CB;
  const int n1 = G > 0 ? (int)((int64_t)(blockIdx.x + 1) * N / G) : min(n0 + 16 * CB, N);

  const int nunits = (K + kUnitK - 1) / kUnitK;
  const int ub = (int)((int64_t)wave * nunits / WAVES);
  const int ue = (int)((int64_t)(wave + 1) * nunits / WAVES);

  // Weight rows n0 .. N-1 and activation rows 0 .. M-1; rows outside read zeros.
  const int64_t wrow = W4 ? K / 2 : K;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (size_t)n0 * (size_t)wrow, (int64_t)(N - n0) * wrow);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, (int64_t)M * K);
  uint32_t wbase[CB], qbase[MB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
    wbase[cb] = (n0 + cb * 16 + col < n1) ? (uint32_t)((cb * 16 + col) * wrow) : kOutOfRange;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) qbase[mb] = (mb * 16 + col < M) ? (uint32_t)((mb * 16 + col) * K) : kOutOfRange;

  // The epilogue scales of this thread's outputs, loaded ahead so that the
  // epilogue does not wait for a memory round trip after the reduction.
  constexpr int kOut = CB * MB * 4 * 64;
  constexpr int kEpt = (kOut + 64 * WAVES - 1) / (64 * WAVES);
  float ea[kEpt], ew[kEpt];
  auto load_scales = [&](bool act) {
#pragma unroll
    for (int t = 0; t < kEpt; ++t) {
      const int e = threadIdx.x + t * 64 * WAVES;
      const int idx = e >> 6, l = e & 63;
      const int m = ((idx / 4) % MB) * 16 + (l >> 4) * 4 + idx % 4;
      const int n = n0 + (idx / (MB * 4)) * 16 + (l & 15);
      const bool ok = e < kOut && m < M && n < n1;
      if (act) ea[t] = ok ? s_a[m] : 0.0f;
      else ew[t] = ok ? s_w[n] : 0.0f;
    }
  };

  v4i acc[CB][MB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[cb][mb] = v4i{0, 0, 0, 0};

  constexpr int WF = W4 ? 1 : 2;  // 16-byte weight fragments per unit and column
  auto load_w = [&](int u0, v4i (&wl)[CB][U][WF]) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int kk = (u0 + j) * kUnitK + g * 32;
      const bool in = (u0 + j < ue) && kk < K;  // K % 32 == 0 (4-bit) keeps a 32-k group whole
      const bool in2 = (u0 + j < ue) && kk + 16 < K;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (W4) {
          wl[cb][j][0] = bload(rw, in ? wbase[cb] + (uint32_t)(kk / 2) : kOutOfRange);
        } else {
          wl[cb][j][0] = bload(rw, in ? wbase[cb] + (uint32_t)kk : kOutOfRange);
          wl[cb][j][WF - 1] = bload(rw, in2 ? wbase[cb] + (uint32_t)(kk + 16) : kOutOfRange);
        }
      }
    }
  };
  auto load_a = [&](int u0, v4i (&al)[MB][U][2]) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int kk = (u0 + j) * kUnitK + g * 32;
      const bool in = (u0 + j < ue) && kk < K;
      const bool in2 = (u0 + j < ue) && kk + 16 < K;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (EARLY) {
          const int row = mb * 16 + col;
          const int8_t* pa = q + row * a_stride + kk;
          al[mb][j][0] = (row < M && in) ? *reinterpret_cast<const v4i*>(pa) : v4i{0, 0, 0, 0};
          al[mb][j][1] = (row < M && in2) ? *reinterpret_cast<const v4i*>(pa + 16) : v4i{0, 0, 0, 0};
        } else {
          al[mb][j][0] = bload(rq, in ? qbase[mb] + (uint32_t)kk : kOutOfRange);
          al[mb][j][1] = bload(rq, in2 ? qbase[mb] + (uint32_t)(kk + 16) : kOutOfRange);
        }
      }
    }
  };
  auto mma = [&](const v4i (&wl)[CB][U][WF], const v4i (&al)[MB][U][2]) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        v4i b0, b1;
        if (W4) {
          unpack_w4(wl[cb][j][0], b0, b1);
        } else {
          b0 = wl[cb][j][0];
          b1 = wl[cb][j][WF - 1];
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc[cb][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al[mb][j][0], b0, acc[cb][mb], 0, 0, 0);
          acc[cb][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al[mb][j][1], b1, acc[cb][mb], 0, 0, 0);
        }
      }
    }
  };

  if constexpr (!EARLY) {
    load_scales(true);
    load_scales(false);
    for (int u0 = ub; u0 < ue; u0 += U) {
      // All loads of the batch first.
      v4i wl[CB][U][WF];
      v4i al[MB][U][2];
      load_w(u0, wl);
      load_a(u0, al);
      // Keep every load of the batch ahead of the first MFMA (the scheduler
      // would otherwise pair each load with its use and wait on it).
      __builtin_amdgcn_sched_barrier(0);
      mma(wl, al);
    }
  } else {
    // The weights of the first batch are requested before the wait for the
    // activations, which then overlaps their latency.  The weight scales are
    // requested after it: a wait for any earlier load would wait for them
    // too (loads complete in order).
    before();
    v4i wl[CB][U][WF];
    load_w(ub, wl);
    wait();
    load_scales(false);
    load_scales(true);
    for (int u0 = ub; u0 < ue; u0 += U) {
      if (u0 != ub) load_w(u0, wl);
      v4i al[MB][U][2];
      load_a(u0, al);
      __builtin_amdgcn_sched_barrier(0);
      mma(wl, al);
    }
  }

#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][(cb * MB + mb) * 4 + i][lane] = acc[cb][mb][i];
  __syncthreads();

  // Output layout of the 16x16 MFMA: lane l, register i -> row 4 * (l / 16) + i,
  // column l % 16.
#pragma unroll
  for (int t = 0; t < kEpt; ++t) {
    const int e = threadIdx.x + t * 64 * WAVES;
    if (e >= kOut) break;
    const int idx = e >> 6;
    const int l = e & 63;
    int s = 0;
#pragma unroll
    for (int wv = 0; wv < WAVES; ++wv) s += red[wv][idx][l];
    if (W4) s >>= 4;  // exact: the sum is a multiple of 16
    const int cb = idx / (MB * 4), mb = (idx / 4) % MB, i = idx % 4;
    const int m = mb * 16 + (l >> 4) * 4 + i;
    const int n = n0 + cb * 16 + (l & 15);
    if (m < M && n < n1) {
      const size_t o = (size_t)m * (size_t)N + (size_t)n;
      if (acc_out) acc_out[o] = s;
      const float v = (float)s * ea[t];
      y[o] = v * ew[t];
    }
  }
}

template <int MB, int CB, bool W4, int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void gemm_small_kernel(const int8_t* __restrict__ q,
                                                                const float* __restrict__ s_a,
                                                                const int8_t* __restrict__ w,
                                                                const float* __restrict__ s_w,
                                                                float* __restrict__ y,
                                                                int32_t* __restrict__ acc_out, int M, int N,
                                                                int K, int G) {
  small_gemm<MB, CB, W4, WAVES, U>(q, s_a, w, s_w, y, acc_out, M, N, K, G);
}

// Quantize + W8A8 GEMM of MR = 2, 3 or 4 rows in one launch, with no
// exchange between workgroups: every workgroup quantizes all MR rows itself
// (the rows are short next to its share of the weights) and keeps the codes
// in LDS, as the single-row fused kernel does.  Order of work: the rows of x
// are loaded (CPT float4 of each row per thread, all in flight at once),
// then the first batch of weights is requested; the row absmax and
// finiteness are reduced over the workgroup, and the codes are written to
// LDS with the quantizer's arithmetic (quant_math.h) while those weights
// are in flight.
// Workgroup 0 also writes the codes and scales to q and s_a, which then hold
// what prism_quantize_rows would write.  The GEMM body then reads the
// activation fragments from LDS.  K <= 4 * 512 * CPT.
// Rows x K up to 30720 (15 float4 per thread): past that the workgroups spend
// longer quantizing than the separate quantizer launch costs (MI355X,
// N x K = 2560 x 9728: M = 3 takes 12.4 us in one kernel against 13.0 in
// two launches, M = 4 took 14.3 against 13.2).  More rows lose for the same
// reason even with short rows: every workgroup reads all M rows of x in
// float32, M K 4 bytes per CU from L2 against M K for the codes the GEMM
// reads after a separate quantizer launch (N x K = 9728 x 2560: 5 rows 12.1
// us against 11.3 in two launches, 8 rows 13.9 against 11.5, 16 rows 21.3
// against 12.0).
constexpr int kFusedFloat4PerThread = 15;
template <int MR>
constexpr int fused_k_max() {
  return 4 * 512 * (kFusedFloat4PerThread / MR);
}

template <int MR, int CB, int U>
__global__ __launch_bounds__(512) void quantize_gemm_small_kernel(const float* __restrict__ x,
                                                                  int8_t* __restrict__ q_out,
                                                                  float* __restrict__ s_out,
                                                                  const int8_t* __restrict__ w,
                                                                  const float* __restrict__ s_w,
                                                                  float* __restrict__ y,
                                                                  int32_t* __restrict__ acc_out, int N, int K,
                                                                  int G) {
  constexpr int WAVES = 8, NT = 512;
  constexpr int CPT = kFusedFloat4PerThread / MR;
  constexpr int KMAX = fused_k_max<MR>();
  __shared__ __attribute__((aligned(16))) int8_t codes[MR * (KMAX + 16)];
  __shared__ float scales[MR];
  __shared__ float rmax[MR][WAVES];
  __shared__ int rfin[MR][WAVES];
  const int stride = K + 16;  // LDS row stride of the codes (K % 16 == 0)
  const int n4 = K / 4;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  float4 v[MR][CPT];

  float amax[MR];
  bool finite[MR];
  // The rows are loaded and this thread's absmax taken before any weight is
  // requested: issued after the weights, the row loads would queue in HBM
  // behind the whole weight stream (every workgroup requests its first
  // batch at once), several microseconds.
  auto load_rows = [&]() {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = threadIdx.x + NT * i;
        if (c < n4) v[m][i] = x4[(size_t)m * (size_t)n4 + (size_t)c];
      }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      amax[m] = 0.0f;
      finite[m] = true;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        if (threadIdx.x + NT * i < n4) {
          amax[m] = fmaxf(amax[m], quant::absmax4(v[m][i]));
          finite[m] = finite[m] && quant::finite4(v[m][i]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto quantize = [&]() {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float a = quant::wave_max(amax[m]);
      const bool f = __all(finite[m]);
      if (lane == 0) {
        rmax[m][wave] = a;
        rfin[m][wave] = f ? 1 : 0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float amax = rmax[m][0];
      int fin = rfin[m][0];
#pragma unroll
      for (int i = 1; i < WAVES; ++i) {
        amax = fmaxf(amax, rmax[m][i]);
        fin &= rfin[m][i];
      }
      const float sc = quant::row_scale(amax, fin != 0);
      const bool zero = fin == 0 || sc == 0.0f;
      const float rc = zero ? 0.0f : quant::fast_recip(sc);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = threadIdx.x + NT * i;
        if (c < n4) {
          const uint32_t code = zero ? 0u : quant::pack4(v[m][i], sc, rc);
          *reinterpret_cast<uint32_t*>(codes + m * stride + 4 * c) = code;
          if (blockIdx.x == 0) reinterpret_cast<uint32_t*>(q_out)[(size_t)m * (size_t)n4 + (size_t)c] = code;
        }
      }
      if (threadIdx.x == 0) {
        scales[m] = sc;
        if (blockIdx.x == 0) s_out[m] = sc;
      }
    }
    __syncthreads();
  };
  small_gemm<1, CB, false, WAVES, U, true>(codes, scales, w, s_w, y, acc_out, MR, N, K, G, load_rows, quantize,
                                           stride);
}

// G > 0: G workgroups with even shares of the N columns (each share at most
// 16 CB columns); G == 0: one workgroup per 16 CB columns.
template <int MB, int CB, bool W4, int WAVES>
void launch_small(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc,
                  int M, int N, int K, int G, hipStream_t st) {
  constexpr int U = MB >= 4 ? 2 : 4;  // units per batch: keeps the batch's registers under ~100 VGPRs
  const unsigned grid = G > 0 ? (unsigned)G : (unsigned)((N + 16 * CB - 1) / (16 * CB));
  gemm_small_kernel<MB, CB, W4, WAVES, U><<<grid, 64 * WAVES, 0, st>>>(q, s_a, w, s_w, y, acc, M, N, K, G);
}

// Column blocks per workgroup and waves per workgroup, from sweeps on MI355X
// (the README's kernels are likewise picked per GPU from measured tables).
// Every choice computes the same exact sums, so this only moves time.
//  * Column blocks c in {1, 2, 3, 4}: the count that minimizes rounds x c,
//    rounds = ceil(ceil(N / 16 / c) / 256), i.e. the workgroups spread evenly
//    over the 256 CUs; ties go to the larger count, whose workgroups read the
//    activations fewer times (each fragment feeds c column blocks), except
//    at M = 1, where a fragment holds one real row and reuse gains nothing
//    (4-bit weights, N = 12288: 7.0 us with one block, 7.1 with three).  At
//    N = 12288 (768 blocks) three blocks give exactly 256 workgroups: 4-bit
//    weights, K = 4096, M = 16 take 8.2 us against 10.5 us with one block,
//    M = 64 15.0 against 23.0 us; N = 9728, K = 2560, int8, M = 16: 8.5 against
//    11.0 us.
//  * Waves: 8 with three or four blocks; with one or two blocks, as measured
//    over six (N, K) shapes x M in {1, 16, 33, 64}: M <= 32: 4-bit weights 8
//    waves once K >= 3072 (four 128-k units per wave), int8 weights 4 waves up
//    to K = 5120 and 8 above; M > 32: 4 waves with two blocks, else 16 waves
//    (N >= 4096) or 8.
int waves_for(int M, int N, int K, bool w4, int cb) {
  const int64_t nunits = (K + kUnitK - 1) / kUnitK;
  if (cb >= 3) return 8;
  if (M <= 32) return w4 ? (nunits >= 24 ? 8 : 4) : (nunits <= 40 ? 4 : 8);
  if (cb == 2) return 4;
  return N >= 4096 ? 16 : 8;
}

void choose_small(int M, int N, int K, bool w4, int& cb, int& waves) {
  // 4-bit weights, 8 or more rows, more than 16384 columns: fewer, wider
  // workgroups re-read the activations fewer times (MI355X, M = 8: 18432
  // columns, 3 blocks: K = 4096 12.4 -> 11.3 us, K = 9728 28.2 -> 24.3 us;
  // 28672 columns, 4 blocks of 4 waves: K = 5120 24.1 -> 19.6 us).
  if (w4 && M >= 8 && N > 16384) {
    cb = N <= 24576 ? 3 : 4;
    waves = cb == 3 ? 8 : 4;
    return;
  }
  const int64_t blocks = (N + 15) / 16;
  int64_t best = -1;
  for (int c = 1; c <= 4; ++c) {
    const int64_t cost = ((blocks + c - 1) / c + 255) / 256 * c;
    if (best < 0 || cost < best || (cost == best && M > 1)) {
      best = cost;
      cb = c;
    }
  }
  waves = waves_for(M, N, K, w4, cb);
}

template <bool W4>
bool pick_variant(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc,
                  int M, int N, int K, int cb, int waves, int G, hipStream_t st) {
#define PRISM_SMALL_CASE(MB)                                                                              \
  if (cb == 1 && waves == 4) launch_small<MB, 1, W4, 4>(q, s_a, w, s_w, y, acc, M, N, K, G, st);           \
  else if (cb == 1 && waves == 8) launch_small<MB, 1, W4, 8>(q, s_a, w, s_w, y, acc, M, N, K, G, st);      \
  else if (cb == 1 && waves == 16) launch_small<MB, 1, W4, 16>(q, s_a, w, s_w, y, acc, M, N, K, G, st);    \
  else if (cb == 2 && waves == 4) launch_small<MB, 2, W4, 4>(q, s_a, w, s_w, y, acc, M, N, K, G, st);      \
  else if (cb == 2 && waves == 8) launch_small<MB, 2, W4, 8>(q, s_a, w, s_w, y, acc, M, N, K, G, st);      \
  else if (cb == 2 && waves == 16) launch_small<MB, 2, W4, 16>(q, s_a, w, s_w, y, acc, M, N, K, G, st);    \
  else if (cb == 3 && waves == 4) launch_small<MB, 3, W4, 4>(q, s_a, w, s_w, y, acc, M, N, K, G, st);      \
  else if (cb == 3 && waves == 8) launch_small<MB, 3, W4, 8>(q, s_a, w, s_w, y, acc, M, N, K, G, st);      \
  else if (cb == 4 && waves == 4) launch_small<MB, 4, W4, 4>(q, s_a, w, s_w, y, acc, M, N, K, G, st);      \
  else if (cb == 4 && waves == 8) launch_small<MB, 4, W4, 8>(q, s_a, w, s_w, y, acc, M, N, K, G, st);      \
  else return false;
  if (M <= 16) { PRISM_SMALL_CASE(1) }
  else if (M <= 32) { PRISM_SMALL_CASE(2) }
  else { PRISM_SMALL_CASE(4) }
#undef PRISM_SMALL_CASE
  return true;
}

// ---------------------------------------------------------------------------
// Small-M block-scale GEMMs (M <= 16): fp16 block scales (Q8_0 style) or the
// Q4_K planes (packed 4-bit codes and 16-byte super-block headers, from which
// D = d * sc and Mn = dmin * m are decoded; both exact in fp32).  The fp32 fold over the
// blocks is a chain in ascending k that cannot be split, but the exact int32
// block sums can: a workgroup owns 16 output columns and walks K in chunks of
// 4 * WAVES blocks.  Phase 1: each wave computes the sums P = sum q * w of
// four consecutive blocks (and for Q4_K S = sum q, from a B operand of ones)
// with v_mfma_i32_16x16x32_i8 (one 32-k block per instruction, lane l holding
// row / column l % 16) into LDS; operands are fetched as 16 bytes per lane,
// 64 contiguous bytes per row and load, and regrouped into one block per
// MFMA with v_permlane32_swap.  Q4_K codes stay packed: 32 bytes hold the
// codes of two sub-blocks (byte l: k = l in the low nibble, k = 32 + l in the
// high one), so the lanes that need k 0-15 and 32-47 of a block pair load the
// same 16 bytes and keep the low or the high nibbles.  Every thread also
// moves one of the chunk's scales into LDS (Q4_K: it decodes sc and m of one
// sub-block from its super-block header).  Phase 2:
// thread (m, n) folds the chunk's blocks into its chain in order,
// f = fmaf((float)P, d, f) (Q4_K: then f = fmaf(-(float)S, Mn, f)).  Chunks
// rotate through RING register sets: the loads of chunk c + RING - 1 are
// issued before chunk c is consumed.
template <bool Q4K, int WAVES, int RING>
__global__ __launch_bounds__(64 * WAVES) void gemm_block_small_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ s_a, const int8_t* __restrict__ w,
    const uint16_t* __restrict__ d16, const uint8_t* __restrict__ hdr, float* __restrict__ y, int M, int N, int K) {
  constexpr int CH = 4 * WAVES;    // blocks per chunk: one scale per thread
  constexpr int PER = CH / WAVES;  // blocks per wave per chunk
  static_assert(WAVES >= 4, "phase 2 needs a thread for each of the 16 x 16 outputs");
  static_assert(RING >= 2 && RING <= 4, "chunk ring depth");
  // Chunk sums and scales, each output's CH values contiguous (padded to CHP
  // so that rows stay 16-byte aligned and consecutive columns fall in
  // different banks): a chain thread reads them with 16-byte loads before its
  // chain of fmas instead of one 4-byte LDS read per step.
  constexpr int CHP = CH + 4;
  __shared__ __attribute__((aligned(16))) int pbuf[16][16][CHP];  // [row][column][block]
  __shared__ __attribute__((aligned(16))) int sbuf[Q4K ? 16 : 1][CHP];  // [row][block]
  __shared__ __attribute__((aligned(16))) float sdv[16][CHP];      // [column][block]
  __shared__ __attribute__((aligned(16))) float smv[Q4K ? 16 : 1][CHP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int NB = K / 32;
  const int col = lane & 15, g = lane >> 4;

  // Bytes per weight row: K int8 codes, or K / 2 packed 4-bit codes.
  const int WR = Q4K ? K / 2 : K;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, (int64_t)M * K);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (size_t)n0 * (size_t)WR, (int64_t)(N - n0) * WR);
  // Rows / columns outside the matrices start out of range and stay there (+ 32 b < 2^31).
  // Blocks past K of an in-range row read the next row's bytes; their sums are never stored.
  // Lane (col, g) loads 16 bytes at 16 g of each 64-byte pair of blocks (Q4_K: at
  // 16 (g % 2) of the pair's 32 packed bytes, low nibbles for g < 2).
  const uint32_t qbase = col < M ? (uint32_t)(col * K + 16 * g) : kOutOfRange;
  const uint32_t wbase = n0 + col < N ? (uint32_t)(col * WR + 16 * (Q4K ? (g & 1) : g)) : kOutOfRange;
  const int nib = (g >> 1) * 4;  // Q4_K: 0 = low nibbles, 4 = high nibbles
  const int64_t ones = 0x0101010101010101LL;
  // Scales of the 16 columns through one buffer resource; this thread moves
  // scale (block tb, column tc) of each chunk, zero past K or past N (Q4_K: the
  // 16-byte header of the block's super-block, of which it decodes one sub-block).
  const int NS = K / 256;
  const int64_t sbytes = Q4K ? (int64_t)(N - n0) * NS * 16 : (int64_t)(N - n0) * NB * 2;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(Q4K ? (const void*)(hdr + (size_t)n0 * NS * 16) : (const void*)(d16 + (size_t)n0 * NB), sbytes);
  // Consecutive threads take consecutive blocks of one column, so a wave's
  // scale load reads a few contiguous runs instead of 16 scattered pieces.
  const int tb = threadIdx.x % CH, tc = threadIdx.x / CH;

  const int pm = threadIdx.x >> 4, pn = threadIdx.x & 15;  // phase-2 output of this thread
  const bool chain = pm < M && n0 + pn < N;
  const float sam = chain ? s_a[pm] : 0.0f;  // loaded early, used once at the end
  float f = 0.0f;

  // A chunk's loads stay raw in registers until the chunk is consumed (Q4_K:
  // packed codes and the header; unpacking them right after the loads would
  // make every chunk wait for its own loads).
  struct Chunk {
    int64_t a[PER], b[PER];
    uint32_t d;  // binary16 bits of the block scale
    v4i h;
  };
  auto load = [&](int b0, Chunk& c) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < PER; j += 2) {
      const int b = b0 + wave * PER + j;
      const v4i x = __builtin_amdgcn_raw_buffer_load_b128(rq, qbase + 32 * b, 0, 0);
      const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rw, wbase + (Q4K ? 16 : 32) * b, 0, 0);
      c.a[j] = ((int64_t)(uint32_t)x[1] << 32) | (uint32_t)x[0];
      c.a[j + 1] = ((int64_t)(uint32_t)x[3] << 32) | (uint32_t)x[2];
      c.b[j] = ((int64_t)(uint32_t)v[1] << 32) | (uint32_t)v[0];
      c.b[j + 1] = ((int64_t)(uint32_t)v[3] << 32) | (uint32_t)v[2];
    }
    const bool sin = b0 + tb < NB && n0 + tc < N;
    if constexpr (Q4K) {
      const uint32_t so = sin ? (uint32_t)(tc * NS + ((b0 + tb) >> 3)) * 16u : kOutOfRange;
      c.h = __builtin_amdgcn_raw_buffer_load_b128(rs, so, 0, 0);
    } else {
      const uint32_t so = sin ? (uint32_t)(tc * NB + b0 + tb) * 2u : kOutOfRange;
      c.d = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
    }
  };
  auto consume = [&](int b0, const Chunk& c) __attribute__((always_inline)) {
    const int nb = NB - b0 < CH ? NB - b0 : CH;
    int64_t av[PER], bv[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      av[j] = c.a[j];
      bv[j] = Q4K ? (int64_t)(((uint64_t)c.b[j] >> nib) & 0x0f0f0f0f0f0f0f0full) : c.b[j];
    }
    // Lanes 0-31 (g = 0, 1) loaded 16 bytes of block j, lanes 32-63 16
    // bytes of block j + 1, as two 8-byte halves av[j] and av[j + 1].  A
    // v_permlane32_swap of av[j + 1] on lanes 0-31 with av[j] on lanes 32-63
    // leaves every lane with one 8-byte slice of block j in av[j] and one of
    // block j + 1 in av[j + 1]; both operands move alike, so lane l holds the
    // same k of A and B and each MFMA below sums exactly one block.
#pragma unroll
    for (int j = 0; j < PER; j += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t& lo = h ? bv[j] : av[j];
        int64_t& hi = h ? bv[j + 1] : av[j + 1];
        const auto s0 = __builtin_amdgcn_permlane32_swap((uint32_t)lo, (uint32_t)hi, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap((uint32_t)(lo >> 32), (uint32_t)(hi >> 32), false, false);
        lo = ((int64_t)s1[0] << 32) | (uint32_t)s0[0];
        hi = ((int64_t)s1[1] << 32) | (uint32_t)s0[1];
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int bl = wave * PER + j;
      const v4i p = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[j], bv[j], v4i{0, 0, 0, 0}, 0, 0, 0);
      if (bl < nb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * g + i < M) pbuf[4 * g + i][col][bl] = p[i];
      }
      if constexpr (Q4K) {
        const v4i sa = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[j], ones, v4i{0, 0, 0, 0}, 0, 0, 0);
        if (bl < nb && col == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * g + i < M) sbuf[4 * g + i][bl] = sa[i];
        }
      }
    }
    if constexpr (Q4K) {
      float d, m;
      q4k_scale_min(c.h, (b0 + tb) & 7, d, m);
      sdv[tc][tb] = d;
      smv[tc][tb] = m;
    } else {
      sdv[tc][tb] = (float)__builtin_bit_cast(_Float16, (uint16_t)c.d);
    }
    __syncthreads();
    if (chain) {
      // Blocks past K (i >= nb) hold stale sums but zero scales: an fma with a
      // zero scale adds a zero and leaves f unchanged (f starts at +0 and never
      // becomes -0), so the chain runs the whole chunk without a branch.
      constexpr int H = 8;  // blocks per batch of reads
#pragma unroll
      for (int i0 = 0; i0 < CH; i0 += H) {
        int pv[H], sv[H];
        float dv[H], mv[H];
#pragma unroll
        for (int i = 0; i < H; i += 4) {
          *reinterpret_cast<v4i*>(pv + i) = *reinterpret_cast<const v4i*>(&pbuf[pm][pn][i0 + i]);
          *reinterpret_cast<v4f*>(dv + i) = *reinterpret_cast<const v4f*>(&sdv[pn][i0 + i]);
          if constexpr (Q4K) {
            *reinterpret_cast<v4i*>(sv + i) = *reinterpret_cast<const v4i*>(&sbuf[pm][i0 + i]);
            *reinterpret_cast<v4f*>(mv + i) = *reinterpret_cast<const v4f*>(&smv[pn][i0 + i]);
          }
        }
#pragma unroll
        for (int i = 0; i < H; ++i) {
          f = __builtin_fmaf((float)pv[i], dv[i], f);
          if constexpr (Q4K) f = __builtin_fmaf(-(float)sv[i], mv[i], f);
        }
      }
    }
    __syncthreads();  // the next chunk reuses the buffers
  };

  // Chunks past K load zero scales (and sums that are never stored); the
  // loop stops at the first chunk past K, the same point for every thread.
  Chunk c[RING];
#pragma unroll
  for (int r = 0; r < RING - 1; ++r) load(r * CH, c[r]);
  for (int b0 = 0; b0 < NB; b0 += RING * CH) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      if (b0 + r * CH >= NB) break;
      load(b0 + (r + RING - 1) * CH, c[(r + RING - 1) % RING]);
      consume(b0 + r * CH, c[r]);
    }
  }
  if (chain) y[(size_t)pm * (size_t)N + (size_t)(n0 + pn)] = f * sam;
}

// ---------------------------------------------------------------------------
// Block-scale and Q4_K GEMMs of 1 to 4 activation rows.  Each fold chain is
// one output, so the kernel for M <= 16 above spends most of a chunk with
// one wave folding 16 M chains between two barriers while the rest wait.
// Here each wave owns R weight rows and walks K on its own, in groups of 256
// k (8 blocks or sub-blocks: one Q4_K super-block) with W groups of loads in
// flight and no workgroup barrier in the loop (the NWV waves of a workgroup
// share only the activation rows, staged into LDS once).  Per group:
//  * the exact sum of every (activation row, weight row, block) comes from
//    16-byte pieces of the weight rows, one piece per lane and load (Q4_K:
//    8 lanes per row and load, each piece holding half of two sub-blocks'
//    nibbles; int8: 16 lanes per row, each piece half a block), with v_dot4
//    against the activation bytes in LDS, and the two halves of a block
//    added from the neighbouring lane; it goes to LDS as fp32 (exact:
//    |P| < 2^24);
//  * lane l decodes the scales of R / 8 blocks of one weight row into LDS
//    (binary16 d; Q4_K: D = d sc and Mn = dmin m from the row's super-block
//    header);
//  * lane c < M R then runs the fold of output (c / R, c % R) over the
//    group's 8 blocks: f = fmaf(P, d, f) per block (Q4_K: f = fmaf(P, D, f),
//    then f = fmaf(-S, Mn, f), with -S the sub-block's activation sum,
//    computed once per workgroup), in ascending block order, as every other
//    kernel.
// The tables are double-buffered, so the next group's sums need not wait for
// this group's fold.  The activation rows (M K bytes) and -S sit in dynamic
// LDS.  Weight rows past N read nothing (out of range) and store nothing.
// Requires K % 256 == 0 and 16-byte aligned q, w and scale arrays.
template <bool Q4K, int R, int MR>
constexpr int gemv_block_tab() {
  // floats per table buffer of one wave: P [MR][R][8], d or D [R][8], Q4_K Mn [R][8]
  return (MR + (Q4K ? 2 : 1)) * R * 8;
}
template <bool Q4K, int R, int MR, int NWV>
size_t gemv_block_lds(int M, int K) {
  return (size_t)M * K + (Q4K ? (size_t)M * K / 8 : 0) + (size_t)NWV * 2 * gemv_block_tab<Q4K, R, MR>() * 4;
}

template <bool Q4K, int R, int MR, int NWV, int W>
__global__ __launch_bounds__(64 * NWV) void gemv_block_kernel(const int8_t* __restrict__ q,
                                                              const float* __restrict__ s_a,
                                                              const int8_t* __restrict__ w,
                                                              const uint16_t* __restrict__ d16,
                                                              const uint8_t* __restrict__ hdr,
                                                              float* __restrict__ y, int M, int N, int K) {
  static_assert(R == 8 || R == 16, "rows per wave");
  static_assert(MR * R <= 64, "one fold chain per lane");
  constexpr int LPR = Q4K ? 8 : 16;   // lanes per row and load (16-byte pieces of a row's group)
  constexpr int LW = R * LPR / 64;    // weight loads per lane per group of 256 k
  constexpr int ND = R / 8;           // blocks whose scales each lane decodes
  constexpr int TS = R * 8;           // floats per [R][8] table
  extern __shared__ __attribute__((aligned(16))) int8_t gv_lds[];
  int8_t* qs = gv_lds;                                                         // activation rows, M K bytes
  float* nsum = reinterpret_cast<float*>(gv_lds + M * K);                      // Q4_K: -S [M][K / 32]
  // The wave index goes through readfirstlane so that the compiler sees it
  // (and the buffer resources built from it) as uniform; a divergent
  // resource makes it loop over the lanes around every buffer load.
  const int lane = threadIdx.x & 63;
  const int wv = NWV == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  float* tab = reinterpret_cast<float*>(gv_lds + M * K + (Q4K ? M * K / 8 : 0)) +
               wv * 2 * gemv_block_tab<Q4K, R, MR>();                          // this wave's [2] buffers
  const int n0 = (blockIdx.x * NWV + wv) * R;
  const int NG = K / 256;  // groups
  const int WR = Q4K ? K / 2 : K;

  // This lane's pieces: load j covers row rl + j * (64 / LPR), piece p of
  // the row's bytes of a group.
  const int rl = lane / LPR;
  const int p = lane % LPR;
  const int gbytes = Q4K ? 128 : 256;  // weight bytes of one row per group
  const int nrows = n0 < N ? N - n0 : 0;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (size_t)(n0 < N ? n0 : 0) * (size_t)WR, (int64_t)nrows * WR);
  uint32_t wofs[LW];
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    const int r = rl + j * (64 / LPR);
    wofs[j] = r < nrows ? (uint32_t)(r * WR + 16 * p) : kOutOfRange;
  }
  // Scales: lane l takes row l / (8 / ND) and decodes its blocks sb .. sb +
  // ND - 1 of each group (int8: loads those ND binary16 scales; Q4_K: loads
  // the row's 16-byte super-block header).
  const int sr = lane / (8 / ND), sb = ND * (lane % (8 / ND));
  const int NS = K / 256;
  const size_t nc = (size_t)(n0 < N ? n0 : 0);
  const __amdgpu_buffer_rsrc_t rs =
      Q4K ? make_rsrc(hdr + nc * NS * 16, (int64_t)nrows * NS * 16)
          : make_rsrc(d16 + nc * (K / 32), (int64_t)nrows * (K / 32) * 2);
  const uint32_t sofs = sr < nrows ? (uint32_t)(sr * NS * 16 + (Q4K ? 0 : 2 * sb)) : kOutOfRange;

  struct Group {
    v4i b[LW];
    v4i h;   // Q4_K: the header
    int d2;  // int8: the ND binary16 scales
  };
  auto issue = [&](int g, Group& c) __attribute__((always_inline)) {
    const bool in = g < NG;
#pragma unroll
    for (int j = 0; j < LW; ++j) c.b[j] = bload(rw, in ? wofs[j] + (uint32_t)(g * gbytes) : kOutOfRange);
    const uint32_t so = in && sofs != kOutOfRange ? sofs + (uint32_t)(16 * g) : kOutOfRange;
    if constexpr (Q4K) c.h = bload(rs, so);
    else if constexpr (ND == 2) c.d2 = __builtin_amdgcn_raw_buffer_load_b32(rs, so, 0, 0);
    else c.d2 = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
  };

  // The first groups' loads go out before the rows are staged.
  Group c[W];
#pragma unroll
  for (int u = 0; u < W; ++u) issue(u, c[u]);
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, (int64_t)M * K);
    for (int i = threadIdx.x; i < M * K / 16; i += 64 * NWV)
      *reinterpret_cast<v4i*>(qs + 16 * i) = bload(rq, (uint32_t)(16 * i));
    __syncthreads();
    if constexpr (Q4K) {
      for (int b = threadIdx.x; b < M * K / 32; b += 64 * NWV) {
        const v4i x0 = *reinterpret_cast<const v4i*>(qs + 32 * b);
        const v4i x1 = *reinterpret_cast<const v4i*>(qs + 32 * b + 16);
        int t = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          t = __builtin_amdgcn_sdot4(x0[e], 0x01010101, t, false);
          t = __builtin_amdgcn_sdot4(x1[e], 0x01010101, t, false);
        }
        nsum[b] = -(float)t;
      }
      __syncthreads();
    }
  }

  // Output of this lane's fold chain: activation row fm, weight row fr.
  const int fm = lane / R, fr = lane % R;
  const bool chain = fm < M;
  float f = 0.0f;
  auto consume = [&](int g, const Group& c, float* tb) __attribute__((always_inline)) {
    float* tp = tb;                 // P [MR][R][8]
    float* td = tb + MR * TS;       // d or D [R][8]
    float* tm = tb + (MR + 1) * TS; // Q4_K: Mn [R][8]
    const int k0 = 256 * g;
    if constexpr (Q4K) {
      // Piece p: half p & 1 of the pair p >> 1 (32 bytes: byte l holds k = l
      // of the pair in its low nibble and k = 32 + l in its high one).
      const int ka = k0 + 64 * (p >> 1) + 16 * (p & 1);
#pragma unroll
      for (int j = 0; j < LW; ++j) {
        v4i lo4, hi4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t v = (uint32_t)c.b[j][e];
          lo4[e] = (int)(v & 0x0f0f0f0fu);
          hi4[e] = (int)((v >> 4) & 0x0f0f0f0fu);
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (m >= M) break;
          const v4i ql = *reinterpret_cast<const v4i*>(qs + m * K + ka);
          const v4i qh = *reinterpret_cast<const v4i*>(qs + m * K + ka + 32);
          int lo = 0, hi = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo = __builtin_amdgcn_sdot4(lo4[e], ql[e], lo, false);
            hi = __builtin_amdgcn_sdot4(hi4[e], qh[e], hi, false);
          }
          // The other half of each sub-block is in lane ^ 1; sub-block p of
          // the group is the low nibbles' sum on even p, the high on odd.
          const int mine = (p & 1) ? hi : lo, other = (p & 1) ? lo : hi;
          const int t = mine + __builtin_amdgcn_mov_dpp(other, 0xB1, 0xF, 0xF, false);
          tp[m * TS + (rl + j * (64 / LPR)) * 8 + p] = (float)t;
        }
      }
#pragma unroll
      for (int e = 0; e < ND; ++e) {
        float D, Mn;
        q4k_scale_min(c.h, sb + e, D, Mn);
        td[sr * 8 + sb + e] = D;
        tm[sr * 8 + sb + e] = Mn;
      }
    } else {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (m >= M) break;
        const v4i qv = *reinterpret_cast<const v4i*>(qs + m * K + k0 + 16 * p);
#pragma unroll
        for (int j = 0; j < LW; ++j) {
          int t = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) t = __builtin_amdgcn_sdot4(c.b[j][e], qv[e], t, false);
          t += __builtin_amdgcn_mov_dpp(t, 0xB1, 0xF, 0xF, false);
          if ((p & 1) == 0) tp[m * TS + (rl + j * (64 / LPR)) * 8 + (p >> 1)] = (float)t;
        }
      }
      const uint32_t d2 = (uint32_t)c.d2;
#pragma unroll
      for (int e = 0; e < ND; ++e)
        td[sr * 8 + sb + e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(d2 >> (16 * e)));
    }
    if (chain) {
      const float* pr = tp + fm * TS + fr * 8;
      const v4f p0 = *reinterpret_cast<const v4f*>(pr);
      const v4f p1 = *reinterpret_cast<const v4f*>(pr + 4);
      const v4f d0 = *reinterpret_cast<const v4f*>(td + fr * 8);
      const v4f d1 = *reinterpret_cast<const v4f*>(td + fr * 8 + 4);
      const float pv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      const float dv[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
      if constexpr (Q4K) {
        const v4f m0 = *reinterpret_cast<const v4f*>(tm + fr * 8);
        const v4f m1 = *reinterpret_cast<const v4f*>(tm + fr * 8 + 4);
        const float* ns = nsum + fm * (K / 32) + 8 * g;
        const v4f s0 = *reinterpret_cast<const v4f*>(ns);
        const v4f s1 = *reinterpret_cast<const v4f*>(ns + 4);
        const float mv[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
        const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          f = __builtin_fmaf(pv[b], dv[b], f);
          f = __builtin_fmaf(sv[b], mv[b], f);
        }
      } else {
#pragma unroll
        for (int b = 0; b < 8; ++b) f = __builtin_fmaf(pv[b], dv[b], f);
      }
    }
  };

  for (int g0 = 0; g0 < NG; g0 += W) {
#pragma unroll
    for (int u = 0; u < W; ++u) {
      if (g0 + u >= NG) break;
      consume(g0 + u, c[u], tab + ((g0 + u) & 1) * gemv_block_tab<Q4K, R, MR>());
      issue(g0 + u + W, c[u]);
    }
  }
  if (chain && fr < nrows) y[(size_t)fm * N + n0 + fr] = f * s_a[fm];
}

// ---------------------------------------------------------------------------
// M = 1 with int8 weights (a single activation row): one output per weight
// row, so no MFMA tile has to cover 16 columns and the rows can be spread
// evenly over all waves of the grid (each CU then reads an equal share of the
// weights).  Wave j owns rows [j N / W, (j + 1) N / W) of the W waves and
// streams each row with fully coalesced 16-byte loads (64 lanes = 1 KB per
// load): lane l takes the 16-byte pieces l, l + 64, ... of the row.  Products
// are summed with v_dot4_i32_i8 into an int32 per lane, then over the wave
// with shuffles (integer addition: exact, any order).  Rows are processed in
// groups of RG, the loads of the next group in flight while the current one
// is summed.  Epilogue as everywhere: y = ((float)acc * s_a[0]) * s_w[n].
// (With 4-bit weights the MFMA kernel is as fast: its rows are half as long.)
//
// FUSED: the row arrives as fp32 x and every workgroup quantizes it itself,
// into LDS, with the quantizer's arithmetic (quant_math.h): absmax over the
// row, s = amax / 127, codes clamp(rint(x / s)).  The x loads go out first
// and the first weight rows right after them, so the quantization runs
// while those weights are in flight.  Workgroup 0 also writes the codes and the
// scale to q and s_a, which then hold what prism_quantize_rows would write.
template <int PL, int RG, bool FUSED>
__global__ __launch_bounds__(256) void gemv_kernel(const float* __restrict__ x, int8_t* __restrict__ q_out,
                                                   float* __restrict__ s_out, const int8_t* __restrict__ q,
                                                   const float* __restrict__ s_a, const int8_t* __restrict__ w,
                                                   const float* __restrict__ s_w, float* __restrict__ y,
                                                   int32_t* __restrict__ acc_out, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * 4;
  const int r0 = (int)(gw * (int64_t)N / nw), r1 = (int)((gw + 1) * (int64_t)N / nw);
  const int nrows = r1 - r0;  // at most 64 (the grid is sized for it)
  const int P = K / 16;       // 16-byte pieces per row, at most 64 * PL

  const float sw = lane < nrows ? s_w[r0 + lane] : 0.0f;  // lane j: scale of row r0 + j
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (size_t)r0 * (size_t)K, (int64_t)nrows * K);
  v4i a[PL];  // the activation bytes of this lane's pieces
  float sa;   // the row scale

  auto load = [&](v4i (&b)[RG][PL], int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int pc = lane + 64 * i;
        b[r][i] = bload(rw, (j0 + r < nrows && pc < P) ? (uint32_t)((j0 + r) * K + 16 * pc) : kOutOfRange);
      }
  };
  auto sum = [&](const v4i (&b)[RG][PL], int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      if (j0 + r >= nrows) break;
      int s = 0;
#pragma unroll
      for (int i = 0; i < PL; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_sdot4(a[i][e], b[r][i][e], s, false);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
      if (lane == j0 + r) {
        const int n = r0 + j0 + r;
        if (acc_out) acc_out[n] = s;
        const float t = (float)s * sa;
        y[n] = t * sw;
      }
    }
  };

  v4i b0[RG][PL], b1[RG][PL];
  if constexpr (FUSED) {
    __shared__ __attribute__((aligned(16))) uint32_t codes[256 * PL];  // K bytes at most
    __shared__ float red_max[4];
    __shared__ int red_fin[4];
    const int nf4 = K / 4;
    const float4* xr = reinterpret_cast<const float4*>(x);
    float4 v[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int f = threadIdx.x + 256 * j;
      v[j] = f < nf4 ? xr[f] : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    load(b0, 0);
    float amax = 0.0f;
    bool finite = true;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      amax = fmaxf(amax, quant::absmax4(v[j]));
      finite = finite && quant::finite4(v[j]);
    }
    amax = quant::wave_max(amax);
    finite = __all(finite);
    const int wave = threadIdx.x >> 6;
    if (lane == 0) {
      red_max[wave] = amax;
      red_fin[wave] = finite ? 1 : 0;
    }
    __syncthreads();
    amax = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));
    finite = (red_fin[0] & red_fin[1] & red_fin[2] & red_fin[3]) != 0;
    sa = quant::row_scale(amax, finite);
    const bool zero = !finite || sa == 0.0f;
    const float rc = zero ? 0.0f : quant::fast_recip(sa);
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int f = threadIdx.x + 256 * j;
      if (f < nf4) {
        const uint32_t c = zero ? 0u : quant::pack4(v[j], sa, rc);
        codes[f] = c;
        if (blockIdx.x == 0) reinterpret_cast<uint32_t*>(q_out)[f] = c;
      }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) s_out[0] = sa;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int pc = lane + 64 * i;
      a[i] = pc < P ? *reinterpret_cast<const v4i*>(codes + 4 * pc) : v4i{0, 0, 0, 0};
    }
  } else {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, K);
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int pc = lane + 64 * i;
      a[i] = bload(rq, pc < P ? (uint32_t)(16 * pc) : kOutOfRange);
    }
    sa = s_a[0];
    load(b0, 0);
  }
  for (int j0 = 0; j0 < nrows; j0 += 2 * RG) {
    load(b1, j0 + RG);
    sum(b0, j0);
    if (j0 + RG >= nrows) break;
    load(b0, j0 + 2 * RG);
    sum(b1, j0 + RG);
  }
}

// Returns false (nothing launched) for rows longer than 16 KB, which the
// MFMA kernel takes.  Two workgroups of 4 waves per CU; one row per group
// from 4 pieces per lane up (the fastest of groups of 1, 2, 4, 8 rows and 1,
// 2, 4 workgroups per CU at N x K = 5120 x 5120, 2560 x 9728, 9728 x 2560 and
// 17408 x 5120 on MI355X).
// x non-null: the fused form (x quantized inside, codes and scale also
// written to q and s_a).
bool launch_gemv(const float* x, int8_t* q_out, float* s_out, const int8_t* q, const float* s_a, const int8_t* w,
                 const float* s_w, float* y, int32_t* acc, int N, int K, hipStream_t st) {
  const int pl = (K / 16 + 63) / 64;
  const int64_t need = (N + 255) / 256;  // <= 64 rows per wave
  // Two workgroups per CU; one when fused with rows over 5 KB, since every
  // workgroup quantizes the whole row again (measured at K = 2560 and 9728).
  const int64_t base = x && pl > 5 ? 256 : 512;
  const unsigned grid = (unsigned)(need > base ? need : base);
#define PRISM_GEMV(PLV, RGV)                                                                                  \
  case PLV:                                                                                                   \
    if (x)                                                                                                    \
      gemv_kernel<PLV, RGV, true><<<grid, 256, 0, st>>>(x, q_out, s_out, nullptr, nullptr, w, s_w, y, acc, N, K); \
    else                                                                                                      \
      gemv_kernel<PLV, RGV, false><<<grid, 256, 0, st>>>(nullptr, nullptr, nullptr, q, s_a, w, s_w, y, acc, N, K); \
    return true;
  switch (pl) {
    PRISM_GEMV(1, 4)
    PRISM_GEMV(2, 2)
    PRISM_GEMV(3, 2)
    PRISM_GEMV(4, 1)
    PRISM_GEMV(5, 1)
    PRISM_GEMV(6, 1)
    PRISM_GEMV(7, 1)
    PRISM_GEMV(8, 1)
    PRISM_GEMV(9, 1)
    PRISM_GEMV(10, 1)
    PRISM_GEMV(11, 1)
    PRISM_GEMV(12, 1)
    PRISM_GEMV(13, 1)
    PRISM_GEMV(14, 1)
    PRISM_GEMV(15, 1)
    PRISM_GEMV(16, 1)
    default:
      return false;
  }
#undef PRISM_GEMV
}

}  // namespace

int launch_gemm_block_small(const int8_t* q, const float* s_a, const int8_t* w, const uint16_t* d16,
                            const uint8_t* hdr, float* y, int M, int N, int K, hipStream_t st) {
  const unsigned grid = (unsigned)((N + 15) / 16);
  // 1 <= M <= 4 rows of at most 16 KB (M = 1) or 32 KB in all, whole
  // super-blocks, aligned scales: the per-wave kernel above.
  if (M <= 4 && K % 256 == 0 && (M == 1 ? K <= 16384 : M * K <= 32768) &&
      (hdr || reinterpret_cast<uintptr_t>(d16) % 16 == 0)) {
    // M = 1: 8 rows per wave in a workgroup of its own (two waves per SIMD
    // at 17408 rows), Q4_K with 6 groups in flight, int8 with 3: the fastest
    // of 8 or 16 rows and 2 to 16 groups at 17408 x 5120 (MI355X: Q4_K 28.5
    // -> 16.0 us against the M <= 16 kernel, block-scale 23.5 -> 20.3 us).
#define PRISM_GEMV_BLOCK(Q4, R, MR, NWV, W)                                                                \
  gemv_block_kernel<Q4, R, MR, NWV, W><<<(unsigned)((N + R * NWV - 1) / (R * NWV)), 64 * NWV,                \
                                        gemv_block_lds<Q4, R, MR, NWV>(M, K), st>>>(                           \
      q, s_a, w, Q4 ? nullptr : d16, Q4 ? hdr : nullptr, y, M, N, K)
    if (M == 1) {
      if (hdr) PRISM_GEMV_BLOCK(true, 8, 1, 1, 6);
      else PRISM_GEMV_BLOCK(false, 8, 1, 1, 3);
    } else {
      if (hdr) PRISM_GEMV_BLOCK(true, 8, 4, 4, 6);
      else PRISM_GEMV_BLOCK(false, 8, 4, 4, 3);
    }
#undef PRISM_GEMV_BLOCK
    return launch_status();
  }
  // 4 waves (16-block chunks), two chunks in flight: the fastest of waves in
  // {4, 8, 16} x ring depth in {2, 3, 4} at 17408 x 5120, M = 1 and 16.
  if (hdr) gemm_block_small_kernel<true, 4, 2><<<grid, 256, 0, st>>>(q, s_a, w, nullptr, hdr, y, M, N, K);
  else gemm_block_small_kernel<false, 4, 2><<<grid, 256, 0, st>>>(q, s_a, w, d16, nullptr, y, M, N, K);
  return launch_status();
}

int launch_gemm_small_variant(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                              float* y, int32_t* acc, int M, int N, int K, int cb, int waves, hipStream_t st, int G) {
  const int8_t* wb = static_cast<const int8_t*>(w);
  const bool ok = w_is_int4 ? pick_variant<true>(q, s_a, wb, s_w, y, acc, M, N, K, cb, waves, G, st)
                            : pick_variant<false>(q, s_a, wb, s_w, y, acc, M, N, K, cb, waves, G, st);
  return ok ? launch_status() : PRISM_ERR_INVALID_ARG;
}

// Even column shares: min(256, N) workgroups (one per CU), each with at most
// 16 cb columns, cb = ceil(ceil(N / 256) / 16) <= 4.
int launch_gemm_small_balanced(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                               float* y, int32_t* acc, int M, int N, int K, hipStream_t st) {
  const int G = N < 256 ? N : 256;
  const int share = (N + G - 1) / G;
  const int cb = (share + 15) / 16;
  if (cb > 4) return PRISM_ERR_INVALID_ARG;
  return launch_gemm_small_variant(q, s_a, w, w_is_int4, s_w, y, acc, M, N, K, cb,
                                   waves_for(M, N, K, w_is_int4, cb), st, G);
}

int launch_gemm_small(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                      float* y, int32_t* acc, int M, int N, int K, hipStream_t st) {
  if (M == 1 && !w_is_int4 &&
      launch_gemv(nullptr, nullptr, nullptr, q, s_a, static_cast<const int8_t*>(w), s_w, y, acc, N, K, st))
    return launch_status();
  int cb, waves;
  choose_small(M, N, K, w_is_int4, cb, waves);
  // Blocks of 16 cb columns that do not fill whole rounds of 256 CUs leave
  // some CUs reading more weight rows than others: then one even share of
  // the columns per CU instead (M <= 16 on MI355X, same bits: int8 2560 x
  // 9728, M = 2: 9.8 -> 8.4 us; 5120 x 5120, M = 4: 9.5 -> 8.6 us; 4-bit
  // 5120 x 5120, M = 1: 7.4 -> 6.2 us; N = 12288, whose 768 blocks already
  // fill the CUs evenly, keeps its blocks).
  const int64_t groups = (N + 16 * cb - 1) / (16 * cb);
  if (groups % 256 != 0 && N <= 16384)
    return launch_gemm_small_balanced(q, s_a, w, w_is_int4, s_w, y, acc, M, N, K, st);
  return launch_gemm_small_variant(q, s_a, w, w_is_int4, s_w, y, acc, M, N, K, cb, waves, st);
}

// Quantize + GEMM of one row in one kernel when the row fits the
// single-row kernel (K <= 16384); otherwise nothing is launched.
bool launch_quantize_gemv(const float* x, int8_t* q, float* s_a, const int8_t* w, const float* s_w, float* y,
                          int32_t* acc, int N, int K, hipStream_t st) {
  return launch_gemv(x, q, s_a, nullptr, nullptr, w, s_w, y, acc, N, K, st);
}

bool launch_quantize_gemm_small(const float* x, int8_t* q, float* s_a, const int8_t* w, const float* s_w, float* y,
                                int32_t* acc, int M, int N, int K, hipStream_t st) {
  if (M < 2 || M > kFusedSmallMMax || N > 16384) return false;
  if (K > (M == 2 ? fused_k_max<2>() : M == 3 ? fused_k_max<3>() : fused_k_max<4>())) return false;
  // One even share of the columns per workgroup, at most one workgroup per
  // CU (as launch_gemm_small_balanced).
  const int G = N < 256 ? N : 256;
  const int cb = ((N + G - 1) / G + 15) / 16;
  // A first batch of two units instead of four for rows up to 4096 (each
  // wave's share of K is then at most four units): the waves that quantize
  // are held up less by their own weight requests (MI355X, N x K = 9728 x
  // 2560, M = 2: 9.8 -> 9.1 us; at K = 9728 four units stay faster).
  const bool u2 = K <= 4096 || cb == 4;
#define PRISM_FUSED(MR, CB)                                                                                    \
  if (M == MR && cb == CB) {                                                                                   \
    if (u2)                                                                                                    \
      quantize_gemm_small_kernel<MR, CB, 2><<<(unsigned)G, 512, 0, st>>>(x, q, s_a, w, s_w, y, acc, N, K, G);  \
    else                                                                                                       \
      quantize_gemm_small_kernel<MR, CB, 4><<<(unsigned)G, 512, 0, st>>>(x, q, s_a, w, s_w, y, acc, N, K, G);  \
    return true;                                                                                               \
  }
  PRISM_FUSED(2, 1) PRISM_FUSED(2, 2) PRISM_FUSED(2, 3) PRISM_FUSED(2, 4)
  PRISM_FUSED(3, 1) PRISM_FUSED(3, 2) PRISM_FUSED(3, 3) PRISM_FUSED(3, 4)
  PRISM_FUSED(4, 1) PRISM_FUSED(4, 2) PRISM_FUSED(4, 3) PRISM_FUSED(4, 4)
#undef PRISM_FUSED
  return false;
}

}  // namespace prism
