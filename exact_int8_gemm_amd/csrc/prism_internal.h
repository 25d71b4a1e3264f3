// Internal declarations shared by the HIP sources of libprism.  Not part of
// the C ABI (that is include/prism.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prism {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Rows up to this count take the split-K small-M kernels; more rows take the
// LDS-tiled kernels.  Either choice gives the same bits (exact int32 sums and
// a fixed per-element epilogue).
constexpr int kSmallMMax = 64;

// Q4_K super-block header (the 16 leading bytes of a GGUF Q4_K super-block,
// as four little-endian dwords: binary16 d and dmin, then the 12 scale bytes
// s[0..11]) -> D = d * sc_j and Mn = dmin * m_j of sub-block j (0..7), both
// exact in fp32 (11 + 6 significant bits).  The 6-bit sc_j and m_j: for
// j < 4, s[j] & 63 and s[j + 4] & 63; for j >= 4, (s[j + 4] & 15) | (s[j - 4]
// >> 6) << 4 and (s[j + 4] >> 4) | (s[j] >> 6) << 4.
__device__ inline void q4k_scale_min(const v4i h, int j, float& D, float& Mn) {
  const int sh = 8 * (j & 3);
  const uint32_t a = ((uint32_t)h[1] >> sh) & 0xffu;  // s[j % 4]
  const uint32_t b = ((uint32_t)h[2] >> sh) & 0xffu;  // s[j % 4 + 4]
  const uint32_t c = ((uint32_t)h[3] >> sh) & 0xffu;  // s[j % 4 + 8]
  const uint32_t sc = j < 4 ? (a & 63u) : ((c & 15u) | ((a >> 6) << 4));
  const uint32_t m = j < 4 ? (b & 63u) : ((c >> 4) | ((b >> 6) << 4));
  const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)((uint32_t)h[0] & 0xffffu));
  const float dmin = (float)__builtin_bit_cast(_Float16, (uint16_t)((uint32_t)h[0] >> 16));
  D = d * (float)sc;
  Mn = dmin * (float)m;
}

// Each launcher assumes its arguments were validated by the C ABI layer and
// returns a PRISM_* status.
int launch_quantize_rows(const float* x, int8_t* q, float* s, int64_t M, int64_t K, hipStream_t st);
int launch_quantize_rows_static(const float* x, int8_t* q, float* s, float scale, int64_t M, int64_t K,
                                hipStream_t st);
// M <= kBlockSmallMMax: block-scale (w int8 codes, d16) or Q4_K (w packed 4-bit
// codes, hdr super-block headers) GEMM of the small-M family.
constexpr int kBlockSmallMMax = 16;
int launch_gemm_block_small(const int8_t* q, const float* s_a, const int8_t* w, const uint16_t* d16,
                            const uint8_t* hdr, float* y, int M, int N, int K, hipStream_t st);
int launch_repack_q4_k(const uint8_t* blocks, uint8_t* w4, uint8_t* hdr, int64_t N, int64_t K, hipStream_t st);
int launch_gemm_q4k(const int8_t* q, const float* s_a, const uint8_t* w4, const uint8_t* hdr, float* y, int M, int N,
                    int K, hipStream_t st);
int launch_repack_q8_0(const uint8_t* blocks, int8_t* w, uint16_t* d, int64_t N, int64_t K, hipStream_t st);

int launch_gemm_small(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                      float* y, int32_t* acc, int M, int N, int K, hipStream_t st);
// One row (M = 1), int8 weights: quantize x and multiply in one kernel, also
// writing the codes to q and the scale to s_a.  False (nothing launched) when
// K is too long for it.
bool launch_quantize_gemv(const float* x, int8_t* q, float* s_a, const int8_t* w, const float* s_w, float* y,
                          int32_t* acc, int N, int K, hipStream_t st);
// 2 <= M <= kFusedSmallMMax rows, N up to 16384, int8 weights: quantize x and
// multiply in one kernel (every workgroup quantizes the rows into LDS, also
// writing the codes to q and the scales to s_a).  False (nothing launched)
// when the shape is outside its range (K up to 14336 for 2 rows, 10240 for
// 3, 6144 for 4).
constexpr int kFusedSmallMMax = 4;
bool launch_quantize_gemm_small(const float* x, int8_t* q, float* s_a, const int8_t* w, const float* s_w, float* y,
                                int32_t* acc, int M, int N, int K, hipStream_t st);

int launch_gemm_tiled(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                      float* y, int32_t* acc, int M, int N, int K, hipStream_t st);

// G > 0: G workgroups with even shares of the N columns, each at most 16 cb.
int launch_gemm_small_variant(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                              float* y, int32_t* acc, int M, int N, int K, int cb, int waves, hipStream_t st,
                              int G = 0);
// The small-M kernel with one even column share per CU (PRISM_ERR_INVALID_ARG
// when a share would exceed 64 columns, i.e. N > 16384).
int launch_gemm_small_balanced(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                               float* y, int32_t* acc, int M, int N, int K, hipStream_t st);
int launch_gemm_tiled_variant(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                              float* y, int32_t* acc, int M, int N, int K, int variant, hipStream_t st);
int launch_gemm_blockscale(const int8_t* q, const float* s_a, const int8_t* w, const uint16_t* d, float* y,
                           int32_t* partials, int M, int N, int K, hipStream_t st);

// Measurement kernels (peaks.hip).
int launch_peak_mfma(int64_t iters, int waves_per_simd, int seed, uint32_t* out, hipStream_t st);
int launch_peak_read(const void* buf, int64_t bytes, uint32_t* parts, int nparts, hipStream_t st);
int launch_peak_fold(int mode, int64_t iters, float* out, hipStream_t st);

// Status of the most recent launch on this thread.
int launch_status();

}  // namespace prism
