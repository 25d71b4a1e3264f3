// Internal declarations shared by the HIP sources of libprism.  Not part of
// the C ABI (that is include/prism.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prism {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Rows up to this count take the split-K small-M kernels; more rows take the
// LDS-tiled kernels.  Either choice gives the same bits (exact int32 sums and
// a fixed per-element epilogue).
constexpr int kSmallMMax = 64;

// Each launcher assumes its arguments were validated by the C ABI layer and
// returns a PRISM_* status.
int launch_quantize_rows(const float* x, int8_t* q, float* s, int64_t M, int64_t K, hipStream_t st);
int launch_quantize_rows_static(const float* x, int8_t* q, float* s, float scale, int64_t M, int64_t K,
                                hipStream_t st);
// M <= kBlockSmallMMax: block-scale (d16) or Q4_K (D, Mn) GEMM of the small-M family.
constexpr int kBlockSmallMMax = 16;
int launch_gemm_block_small(const int8_t* q, const float* s_a, const int8_t* w, const uint16_t* d16,
                            const float* D, const float* Mn, float* y, int M, int N, int K, hipStream_t st);
int launch_repack_q4_k(const uint8_t* blocks, int8_t* w, float* D, float* Mn, int64_t N, int64_t K, hipStream_t st);
int launch_gemm_q4k(const int8_t* q, const float* s_a, const int8_t* w, const float* D, const float* Mn, float* y,
                    int M, int N, int K, hipStream_t st);
int launch_repack_q8_0(const uint8_t* blocks, int8_t* w, uint16_t* d, int64_t N, int64_t K, hipStream_t st);

int launch_gemm_small(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                      float* y, int32_t* acc, int M, int N, int K, hipStream_t st);
// One row (M = 1), int8 weights: quantize x and multiply in one kernel, also
// writing the codes to q and the scale to s_a.  False (nothing launched) when
// K is too long for it.
bool launch_quantize_gemv(const float* x, int8_t* q, float* s_a, const int8_t* w, const float* s_w, float* y,
                          int32_t* acc, int N, int K, hipStream_t st);

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

// Status of the most recent launch on this thread.
int launch_status();

}  // namespace prism
