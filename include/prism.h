/*
 * prism.h -- C ABI of the exact, batch-invariant int8 linear layer for
 * MI355X (gfx950).
 *
 * The operation (StartLux-Prism README): "Why StartLux-Prism" says that the
 * int8 GEMMs sum exactly in int32, so that a request gets the same result
 * whatever it is batched with, and that Q8_0 weights run as int8 (W8A8)
 * while Q4_K_M weights run on their own 4-bit values (W4A8); "How it works"
 * repeats that the int8 tensor-core path sums exactly in int32; "Quick
 * start" says the activations are quantized to int8 with measured ranges.
 * The pages fix neither the activation scale nor the epilogue; the readings
 * taken here are stated at each call below.
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer (HBM of the current HIP
 *     device).  The caller allocates and owns all buffers; the library keeps
 *     no pointer after the call returns and allocates nothing.
 *   - Matrices are dense and row-major with no padding: x, q are [M][K],
 *     w is [N][K], w4 is [N][K/2], d is [N][K/32], y and acc are [M][N],
 *     partials is [M][N][K/32].
 *   - x, q, w and w4 must be 16-byte aligned; every other pointer must be
 *     aligned to its element size.
 *   - Work is enqueued on `stream` (a hipStream_t; 0 = the null stream) and
 *     the call returns without synchronizing.  Results are ready when the
 *     stream reaches that point.
 *   - M = 0 is a successful no-op that touches no memory.
 *   - Arguments are validated before any HIP call; an invalid call returns a
 *     negative status, enqueues nothing and writes nothing.
 *   - Results are a pure function of the inputs: they do not depend on M,
 *     on a row's position in the batch, on the stream or on concurrency.
 *     Calls hold no global state except per-device caches of the device's
 *     architecture and compute-unit count, and may be made from several
 *     threads at once.
 */
#ifndef PRISM_H
#define PRISM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bumped on any change of a signature or of the semantics below. */
#define PRISM_ABI_VERSION 13

/* Largest accepted K.  For K <= 131040 every exact sum of K products of two
 * int8 values (|q|, |w| <= 128) lies strictly inside the int32 range. */
#define PRISM_K_MAX 131040

/* Status codes. */
#define PRISM_OK 0
#define PRISM_ERR_INVALID_ARG (-1) /* null required pointer, negative size, N or K = 0 with M > 0, K > PRISM_K_MAX */
#define PRISM_ERR_ALIGNMENT (-2)   /* misaligned pointer, or K not a multiple of 16 (32 for block-scale and W4A8, 256 for Q4_K) */
#define PRISM_ERR_UNSUPPORTED (-3) /* the current device is not gfx950, or no device is usable */
#define PRISM_ERR_LAUNCH (-4)      /* the kernel launch reported an error */

/* Returns PRISM_ABI_VERSION of the built library. */
int prism_abi_version(void);

/* Identity of the sources the library was built from: 32 hex digits of the
 * sha256 of its HIP/C++ sources, this header and its compile flags (static
 * string, never NULL).  A binding can compare it with the sources it ships
 * with and refuse a library built from others. */
const char* prism_build_id(void);

/* Static, human-readable text for a status code (never NULL). */
const char* prism_status_string(int status);

/*
 * Per-row int8 activation quantizer (README "Quick start": int8 activation
 * ranges; the per-row absmax form is the reading taken here).
 *   x      [M][K] fp32, input.
 *   q      [M][K] int8, output.
 *   scale  [M] fp32, output.
 * For each row m: a = max_k |x[m][k]|; scale[m] = a / 127 (IEEE division,
 * round to nearest even); q[m][k] = clamp(rint(x[m][k] / scale[m]), -127, 127)
 * with rint rounding half to even.  A row holding a NaN or an infinity gets
 * scale NaN and q = 0; a row whose scale is 0 (all zeros, or a subnormal
 * amax that underflows) gets q = 0.  Rows never influence each other.
 * K must be a multiple of 16.
 */
int prism_quantize_rows(const float* x, int8_t* q, float* scale,
                        int64_t M, int64_t K, void* stream);

/*
 * Int8 activation quantizer with one static, calibrated scale for the whole
 * tensor (README "Quick start": the int8 activation ranges are measured once
 * ahead of time, not per batch).
 *   x      [M][K] fp32, input.
 *   q      [M][K] int8, output.
 *   scale  [M] fp32, output: the row scales to hand to the GEMM calls.
 *   s      the calibrated scale, a host value; must be finite and > 0
 *          (otherwise PRISM_ERR_INVALID_ARG and nothing is enqueued).
 * For each row m without a NaN: scale[m] = s and q[m][k] = clamp(rint(x[m][k]
 * / s), -127, 127) (IEEE division, rint half to even), so values beyond the
 * calibrated range saturate at +-127, an infinite x included.  A row holding
 * a NaN gets scale NaN and q = 0.  Rows never influence each other.
 * K must be a multiple of 16; x and q 16-byte aligned, scale 4-byte aligned.
 */
int prism_quantize_rows_static(const float* x, int8_t* q, float* scale, float s,
                               int64_t M, int64_t K, void* stream);

/*
 * Q8_0 weight blocks -> the (w, d) planes of prism_gemm_w8a8_blockscale
 * (README "Why StartLux-Prism": released Q8_0 files run as int8 W8A8 with no
 * conversion step).  The block layout is the public GGUF one, not given by
 * the pages: 34 bytes per block, a little-endian binary16 scale followed by
 * the 32 int8 codes of k = 32 b .. 32 b + 31 of weight row n; blocks are
 * stored row by row, block n * (K/32) + b.
 *   blocks [N * K/32][34] bytes, input (16-byte aligned).
 *   w      [N][K] int8, output: the codes (16-byte aligned).
 *   d      [N][K/32] binary16 bit patterns, output: the scales (2-byte aligned).
 * Pure byte movement: every output equals an input byte pair or byte.
 * K must be a positive multiple of 32; N = 0 is a no-op.
 */
int prism_repack_q8_0(const uint8_t* blocks, int8_t* w, uint16_t* d,
                      int64_t N, int64_t K, void* stream);

/*
 * Q4_K weight super-blocks -> the planes of prism_gemm_w4a8_q4k (README "Why
 * StartLux-Prism": released Q4_K_M files run on their own 4-bit values).  The
 * super-block layout is the public GGUF one, not given by the pages: 144
 * bytes per 256 consecutive weights of one row: binary16 d and dmin
 * (little-endian), 12 bytes of 6-bit sub-block scales sc_j and mins m_j
 * (j < 4: sc_j = s[j] & 63, m_j = s[j+4] & 63; j >= 4: sc_j = (s[j+4] & 15) |
 * (s[j-4] >> 6) << 4, m_j = (s[j+4] >> 4) | (s[j] >> 6) << 4), then 128 bytes of
 * codes (byte 32 g + l: weight 64 g + l in the low nibble, 64 g + 32 + l in
 * the high one).  Weight = d * sc_j * code - dmin * m_j.
 *   blocks [N * K/256][144] bytes, input (16-byte aligned).
 *   w4     [N][K/2] bytes, output: the 128 code bytes of each super-block, in
 *          the file's own order (super-block t of row n at bytes 128 t ..
 *          128 t + 127 of row n); still 4 bits per weight (16-byte aligned).
 *   hdr    [N][K/256][16] bytes, output: the 16 leading bytes of each
 *          super-block (d, dmin, the 12 scale bytes) (16-byte aligned).
 * Pure byte movement: the two planes hold every byte of the blocks once.
 * K must be a positive multiple of 256; N = 0 is a no-op.
 */
int prism_repack_q4_k(const uint8_t* blocks, uint8_t* w4, uint8_t* hdr,
                      int64_t N, int64_t K, void* stream);

/*
 * W4A8 on Q4_K weights (the planes of prism_repack_q4_k).
 *   q [M][K] int8, s_a [M] fp32, w4 [N][K/2] packed codes, hdr [N][K/256][16].
 *   y [M][N] fp32 output.
 * For sub-block b (32 k) of super-block t = b / 8, j = b % 8: D = d * sc_j and
 * Mn = dmin * m_j from the super-block's header (both exact in fp32);
 * P_b = sum q[m][k] * code[n][k] and S_b = sum q[m][k], both exact integers;
 * f = +0; for b ascending: f = fmaf((float)P_b, D, f); f = fmaf(-(float)S_b,
 * Mn, f); then y[m][n] = f * s_a[m].
 * K must be a multiple of 256; q, w4 and hdr 16-byte aligned.
 */
int prism_gemm_w4a8_q4k(const int8_t* q, const float* s_a, const uint8_t* w4, const uint8_t* hdr,
                        float* y, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * W8A8 GEMM with per-output-channel weight scales (README "Why
 * StartLux-Prism": Q8_0 weights as int8 W8A8, summed exactly in int32).
 *   q    [M][K] int8 activations, s_a [M] fp32 row scales.
 *   w    [N][K] int8 weights (one row per output channel), s_w [N] fp32.
 *   y    [M][N] fp32 output.
 *   acc  [M][N] int32 output, or NULL.
 * acc[m][n] = sum_k q[m][k] * w[n][k], exact in int32;
 * y[m][n]   = ((float)acc[m][n] * s_a[m]) * s_w[n], each product rounded
 * to nearest even on its own, in that order.  K must be a multiple of 16.
 */
int prism_gemm_w8a8(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w,
                    float* y, int32_t* acc, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * W8A8 GEMM with one fp16 weight scale per 32 consecutive k of each weight
 * row (Q8_0-style blocks; README "Why StartLux-Prism", released Q8_0 files).
 *   q [M][K] int8, s_a [M] fp32, w [N][K] int8.
 *   d [N][K/32] binary16 bit patterns: the scale of block b of row n.
 *   y [M][N] fp32 output.
 *   partials [M][N][K/32] int32 output, or NULL (meant for small debug sizes).
 * P_b = sum_{32b <= k < 32b+32} q[m][k] * w[n][k] (exact int32);
 * f = +0; for b = 0, 1, ..., K/32-1 in that order: f = fmaf((float)P_b,
 * (float)d[n][b], f); y[m][n] = f * s_a[m].  K must be a multiple of 32.
 */
int prism_gemm_w8a8_blockscale(const int8_t* q, const float* s_a, const int8_t* w,
                               const uint16_t* d, float* y, int32_t* partials,
                               int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Quantize + W8A8 GEMM in one call (the README's "Quick start" int8
 * activations feeding the exact int32 GEMM of "Why StartLux-Prism").
 *   x     [M][K] fp32 activations (16-byte aligned).
 *   q     [M][K] int8 and scale [M] fp32 outputs: what prism_quantize_rows
 *         writes for x.
 *   w, s_w, y, acc: as for prism_gemm_w8a8 (acc may be NULL).
 * The results are those of prism_quantize_rows(x) followed by
 * prism_gemm_w8a8 on its outputs, bit for bit.  With M = 1 and K <= 16384,
 * and with M = 2, 3 or 4 rows, N <= 16384 and K up to 14336, 10240 or 6144
 * respectively, this is one kernel in which every workgroup quantizes the
 * rows on chip while its first weight rows stream in (decode); otherwise
 * the two steps run as two launches on `stream`.  Either way it allocates
 * nothing.  K must be a multiple of 16.
 */
int prism_quantize_gemm_w8a8(const float* x, int8_t* q, float* scale, const int8_t* w, const float* s_w,
                             float* y, int32_t* acc, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * W4A8 GEMM on packed signed 4-bit weights (README "Why StartLux-Prism":
 * Q4_K_M files run on their own 4-bit weights with int8 activations; the
 * symmetric per-channel form is the reading taken here).
 *   q [M][K] int8, s_a [M] fp32.
 *   w4 [N][K/2] bytes: byte j of row n holds w[n][2j] in its low nibble and
 *      w[n][2j+1] in its high nibble, each a two's-complement value in [-8, 7].
 *   s_w [N] fp32, y [M][N] fp32, acc [M][N] int32 or NULL.
 * acc and y as for prism_gemm_w8a8 with w decoded from the nibbles.
 * K must be a multiple of 32.
 */
int prism_gemm_w4a8(const int8_t* q, const float* s_a, const uint8_t* w4, const float* s_w,
                    float* y, int32_t* acc, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The shape-dependent kernel choice of prism_gemm_w8a8 / prism_gemm_w4a8,
 * one entry at a time (README "Why StartLux-Prism": kernels are picked per
 * GPU from measured tables; that is safe here because every entry computes
 * the same exact int32 sums and the same per-element epilogue).  These calls
 * exist to verify that claim: the result of every applicable variant is bit
 * for bit the result of PRISM_VARIANT_AUTO, which is what the plain calls run.
 * Same arguments and checks as the plain calls, plus `variant`:
 *   PRISM_VARIANT_AUTO            the plain call's choice;
 *   PRISM_VARIANT_SMALL_<c>x<w>   the small-M kernel with c column blocks of
 *                                 16 (c = 1..4) and w waves per workgroup
 *                                 (M <= 64 only);
 *   PRISM_VARIANT_SMALL_BALANCED  the small-M kernel with one even share of
 *                                 the N columns per CU (M <= 64, N <= 16384);
 *   PRISM_VARIANT_TILE_*          the LDS-tiled kernels: 256x128, 192x128
 *                                 and 128x96 (int8 weights only), 256x192,
 *                                 256x256, 256x320, 128x128 and 64x128, and
 *                                 128x128 or 64x128 with K split over 2, 3 or
 *                                 4 workgroups, 128x96 over 2, whose exact
 *                                 int32 partials are added atomically into y.
 * A variant that does not apply to the call returns PRISM_ERR_INVALID_ARG.
 */
#define PRISM_VARIANT_AUTO 0
#define PRISM_VARIANT_SMALL_1x4 1
#define PRISM_VARIANT_SMALL_1x8 2
#define PRISM_VARIANT_SMALL_1x16 3
#define PRISM_VARIANT_SMALL_2x4 4
#define PRISM_VARIANT_SMALL_2x8 5
#define PRISM_VARIANT_SMALL_2x16 6
#define PRISM_VARIANT_TILE_256x256 7
#define PRISM_VARIANT_TILE_256x128 8
#define PRISM_VARIANT_TILE_128x128 9
#define PRISM_VARIANT_TILE_128x128_SPLIT2 10
#define PRISM_VARIANT_TILE_128x128_SPLIT3 11
#define PRISM_VARIANT_TILE_128x128_SPLIT4 12
#define PRISM_VARIANT_SMALL_3x4 13
#define PRISM_VARIANT_SMALL_3x8 14
#define PRISM_VARIANT_SMALL_4x4 15
#define PRISM_VARIANT_SMALL_4x8 16
#define PRISM_VARIANT_TILE_256x192 17
#define PRISM_VARIANT_TILE_256x320 18
#define PRISM_VARIANT_TILE_64x128 19
#define PRISM_VARIANT_TILE_64x128_SPLIT2 20
#define PRISM_VARIANT_TILE_64x128_SPLIT3 21
#define PRISM_VARIANT_TILE_64x128_SPLIT4 22
#define PRISM_VARIANT_TILE_128x96 23
#define PRISM_VARIANT_TILE_128x96_SPLIT2 24
#define PRISM_VARIANT_SMALL_BALANCED 25
#define PRISM_VARIANT_TILE_192x128 26
#define PRISM_VARIANT_COUNT 27

int prism_gemm_w8a8_variant(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w,
                            float* y, int32_t* acc, int64_t M, int64_t N, int64_t K, int variant,
                            void* stream);
int prism_gemm_w4a8_variant(const int8_t* q, const float* s_a, const uint8_t* w4, const float* s_w,
                            float* y, int32_t* acc, int64_t M, int64_t N, int64_t K, int variant,
                            void* stream);

/*
 * Measurement kernels (not part of the GEMM path): what this GPU reaches on
 * the two resources the GEMMs are bound by, for the roofline figures.
 *
 * prism_peak_mfma: 2 x (compute units) workgroups, each of 2 x
 * waves_per_simd waves (waves_per_simd in {1, 2, 4}), every wave running
 * iters x 16 v_mfma_i32_32x32x32_i8 on register operands: iters x 16 x 65536
 * integer ops per wave.  out [2 x CUs x 128 x waves_per_simd] uint32 gets
 * one checksum per thread: the sum modulo 2^32 of the thread's NACC x 16
 * accumulator registers after 16 / NACC steps per iteration on NACC
 * accumulators (NACC = 8, or 4 for waves_per_simd = 4) that alternate the
 * operand pairs (A0, B0) and (A1, B1).  Byte j (0..15) of the fragment of
 * operand s (A0, B0, A1, B1 = 0, 1, 2, 3) in lane l is the top byte of
 * (37 l + 101 j + 7919 s + 13 seed) * 2654435761 modulo 2^32, as int8.
 * iters in [1, 2^24], seed in [0, 2^20]; accumulators wrap past 2^31 for
 * large iters (the checksum is then only a data dependence).
 *
 * prism_peak_read: reads `bytes` (a multiple of 16, at most 2^40) of `buf`
 * (16-byte aligned) once with 16-byte loads and writes the XOR of the
 * 32-bit words each workgroup read to parts[workgroup]; all
 * PRISM_PEAK_READ_PARTS entries of parts are written (unused ones 0), so the
 * XOR of parts is the XOR of every 32-bit word of the buffer.
 *
 * prism_peak_fold: the cost of the block-scale fold (an exact sum per 32-k
 * block of a 32 x 32 output tile, then one fp32 fmaf per output,
 * StartLux-Prism README, "Why StartLux-Prism": Q8_0 weights as W8A8) on
 * registers only.  One workgroup of 8 waves per compute unit; each wave
 * holds 5 tiles and gives each one 32-k block per iteration.  mode 0: int8
 * MFMA from zero, convert, fold; 1: two f16 MFMAs on the same values (the
 * sum exact in fp32, no convert), fold; 2: the int8 MFMAs only
 * (accumulating); 3: the f16 MFMA pairs only (accumulating); 4: the folds
 * only.  out [CUs x 512] float gets one sum per thread.  Modes 0 and 1
 * write the same bits; so do modes 2 and 3 for iters <= 32.  iters in [1,
 * 2^20].
 */
#define PRISM_PEAK_READ_PARTS 4096
int prism_peak_mfma(int64_t iters, int waves_per_simd, int seed, uint32_t* out, void* stream);
int prism_peak_read(const void* buf, int64_t bytes, uint32_t* parts, void* stream);
int prism_peak_fold(int mode, int64_t iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PRISM_H */
