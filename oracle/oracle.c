/*
 * oracle.c -- plain, slow CPU oracle for the exact int8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this file.  The GPU
 * library never links it, and it shares no code, header, table or helper
 * with the GPU library.
 *
 * What it computes (StartLux-Prism README):
 *   - "Why StartLux-Prism", bullet on bit reproducibility, and "How it works",
 *     bullet on int8 tensor cores: int8 x int8 products are summed exactly in
 *     int32, so a row's result does not depend on the rows batched with it.
 *   - "Why StartLux-Prism", bullet on the released files: Q8_0 weights run as
 *     int8 (W8A8), Q4_K_M weights on their own 4-bit values (W4A8).
 *   - "Quick start": int8 activation ranges (here: per-row absmax, read below).
 *
 * Every sum is an int64 triple loop (m, n, k); int64 cannot overflow for the
 * accepted K, and the int32 range is then checked explicitly.  The fp32
 * epilogues are written as separate statements so that each operation is
 * rounded on its own (compile with -ffp-contract=off).
 *
 * Readings where the pages say nothing (each is listed in the design notes):
 *   R1 activation scale: per row, s = max|x| / 127 (IEEE fp32 division);
 *      q = clamp(rint(x / s), -127, 127), rint = round half to even.
 *   R2 a row with a non-finite entry gets s = NaN and q = 0; a row whose
 *      scale is 0 (all zeros, or an amax that underflows when divided by 127)
 *      gets q = 0 and keeps that scale.
 *   R3 per-channel epilogue: y = ((float)acc * s_a[m]) * s_w[n], two
 *      separately rounded products, left to right.
 *   R4 block-scale epilogue: f = +0; for b ascending f = fmaf((float)P_b,
 *      (float)d[n][b], f); y = f * s_a[m].
 *   R5 4-bit weights: two's-complement nibbles in [-8, 7], two per byte
 *      along K, the low nibble holds the even k.
 *   R7 Q8_0 weight blocks (the public GGUF layout; the pages only say that
 *      Q8_0 files run as int8 with no conversion step): 34 bytes per block,
 *      a little-endian binary16 scale then the 32 int8 codes of k = 32 b ..
 *      32 b + 31 of row n; blocks follow each other row by row, block
 *      n * (K / 32) + b.  A block stands for the values scale * code, which
 *      is exactly the block-scale operand pair (w, d) of R4.
 *   R8 Q4_K weight blocks (the public GGUF layout; the pages only say that
 *      Q4_K_M files run on their own 4-bit values): a super-block of 256
 *      weights in 144 bytes: binary16 d, binary16 dmin (little-endian), 12
 *      bytes of 6-bit sub-block scales sc_j and mins m_j (j = 0..7: for j < 4
 *      sc_j = s[j] & 63, m_j = s[j+4] & 63; for j >= 4 sc_j = (s[j+4] & 15) |
 *      (s[j-4] >> 6) << 4, m_j = (s[j+4] >> 4) | (s[j] >> 6) << 4), then 128
 *      bytes of codes: byte 32 g + l holds the code of weight 64 g + l in its
 *      low nibble and of weight 64 g + 32 + l in its high nibble.  Weight =
 *      d sc_j code - dmin m_j.  Per 32-weight sub-block the sums P = sum
 *      code * a and S = sum a are exact integers, D = d * sc_j and Mn = dmin
 *      * m_j are exact in fp32, and f = +0; for each sub-block in ascending
 *      k: f = fmaf((float)P, D, f); f = fmaf(-(float)S, Mn, f); y = f * s_a.
 *   R9 Q4_K planes for the GPU GEMM: the file's 128 code bytes of each
 *      super-block, in their own order, form the row's packed codes (K/2
 *      bytes per row, still 4 bits per weight), and its 16 leading bytes (d,
 *      dmin, scales) form a separate header plane.
 *   R6 static activation scale ("Quick start": ranges measured once, ahead
 *      of time): one fp32 s > 0 for the whole tensor; q = clamp(rint(x / s),
 *      -127, 127) saturates values beyond the calibrated range (an infinite
 *      x gives +-127); a row holding a NaN gets scale NaN and q = 0, every
 *      other row gets scale s.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_RANGE (-5) /* an exact sum left the int32 range */

static const int64_t INT32_LIMIT = 2147483648LL; /* 2^31 */

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* IEEE 754 binary16 -> binary32, from the format's definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits.  Every binary16 value is
 * exactly representable in binary32, so the conversion is exact. */
float oracle_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    float v;
    if (e == 0x1f) {
        v = (f == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        v = ldexpf((float)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    } else {
        v = ldexpf((float)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

void oracle_f16_to_f32_array(const uint16_t* h, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f32(h[i]);
}

/* Decode one signed 4-bit weight (R5). */
static int oracle_w4_at(const uint8_t* row, int64_t k) {
    uint8_t byte = row[k / 2];
    int nib = (k % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
    return nib >= 8 ? nib - 16 : nib;
}

/* Per-row activation quantizer (R1, R2). */
int oracle_quantize_rows(const float* x, int8_t* q, float* s, int64_t M, int64_t K) {
    if (M < 0 || K <= 0 || (M > 0 && (!x || !q || !s))) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const float* xr = x + m * K;
        int8_t* qr = q + m * K;
        int finite = 1;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (!isfinite(xr[k])) finite = 0;
            float a = fabsf(xr[k]);
            if (a > amax) amax = a;
        }
        if (!finite) {
            s[m] = NAN;
            memset(qr, 0, (size_t)K);
            continue;
        }
        float sc = amax / 127.0f;
        s[m] = sc;
        if (sc == 0.0f) {
            memset(qr, 0, (size_t)K);
            continue;
        }
        for (int64_t k = 0; k < K; ++k) {
            float t = xr[k] / sc;
            float r = nearbyintf(t); /* default rounding mode: half to even */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            qr[k] = (int8_t)r;
        }
    }
    return ORACLE_OK;
}

/* Activation quantizer with one static scale for the tensor (R6). */
int oracle_quantize_rows_static(const float* x, int8_t* q, float* s, float scale, int64_t M, int64_t K) {
    if (M < 0 || K <= 0 || (M > 0 && (!x || !q || !s))) return ORACLE_ERR_ARG;
    if (!(scale > 0.0f) || isinf(scale)) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const float* xr = x + m * K;
        int8_t* qr = q + m * K;
        int has_nan = 0;
        for (int64_t k = 0; k < K; ++k)
            if (isnan(xr[k])) has_nan = 1;
        if (has_nan) {
            s[m] = NAN;
            memset(qr, 0, (size_t)K);
            continue;
        }
        s[m] = scale;
        for (int64_t k = 0; k < K; ++k) {
            float t = xr[k] / scale;
            float r = nearbyintf(t); /* half to even; +-inf stays +-inf */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            qr[k] = (int8_t)r;
        }
    }
    return ORACLE_OK;
}

/* Q8_0 blocks -> int8 codes w [N][K] and binary16 scale bits d [N][K/32] (R7). */
int oracle_repack_q8_0(const uint8_t* blocks, int8_t* w, uint16_t* d, int64_t N, int64_t K) {
    if (N < 0 || K <= 0 || K % 32 != 0 || (N > 0 && (!blocks || !w || !d))) return ORACLE_ERR_ARG;
    const int64_t NB = K / 32;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < NB; ++b) {
            const uint8_t* blk = blocks + (n * NB + b) * 34;
            d[n * NB + b] = (uint16_t)(blk[0] | (blk[1] << 8));
            for (int64_t j = 0; j < 32; ++j) w[n * K + b * 32 + j] = (int8_t)blk[2 + j];
        }
    }
    return ORACLE_OK;
}

/* Q4_K super-block helpers (R8). */
static void oracle_q4k_scale_min(const uint8_t* sb, int j, int* sc, int* mn) {
    const uint8_t* s = sb + 4;
    if (j < 4) {
        *sc = s[j] & 63;
        *mn = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

static int oracle_q4k_code(const uint8_t* sb, int i) { /* i = 0..255 within the super-block */
    const uint8_t* qs = sb + 16;
    const int g = i / 64, l = i % 64;
    return l < 32 ? (qs[32 * g + l] & 15) : (qs[32 * g + l - 32] >> 4);
}

/* Q4_K blocks -> the two planes the GPU GEMM reads (R9): the 128 code bytes of
 * each super-block, in the file's own order, to w4 [N][K/2] (super-block t of
 * row n at bytes 128 t .. 128 t + 127 of row n), and its first 16 bytes (d,
 * dmin and the 12 scale bytes) to hdr [N][K/256][16].  Pure byte movement. */
int oracle_repack_q4_k(const uint8_t* blocks, uint8_t* w4, uint8_t* hdr, int64_t N, int64_t K) {
    if (N < 0 || K <= 0 || K % 256 != 0 || (N > 0 && (!blocks || !w4 || !hdr))) return ORACLE_ERR_ARG;
    const int64_t NS = K / 256;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t t = 0; t < NS; ++t) {
            const uint8_t* sb = blocks + (n * NS + t) * 144;
            for (int i = 0; i < 16; ++i) hdr[(n * NS + t) * 16 + i] = sb[i];
            for (int i = 0; i < 128; ++i) w4[n * (K / 2) + t * 128 + i] = sb[16 + i];
        }
    }
    return ORACLE_OK;
}

/* W4A8 on Q4_K blocks (R8), straight from the blocks. */
int oracle_gemm_w4a8_q4k(const int8_t* q, const float* s_a, const uint8_t* blocks, float* y,
                         int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N <= 0 || K <= 0 || K % 256 != 0) return ORACLE_ERR_ARG;
    if (M > 0 && (!q || !s_a || !blocks || !y)) return ORACLE_ERR_ARG;
    const int64_t NS = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float f = 0.0f;
            for (int64_t t = 0; t < NS; ++t) {
                const uint8_t* sb = blocks + (n * NS + t) * 144;
                const float d = oracle_f16_to_f32((uint16_t)(sb[0] | (sb[1] << 8)));
                const float dmin = oracle_f16_to_f32((uint16_t)(sb[2] | (sb[3] << 8)));
                for (int j = 0; j < 8; ++j) {
                    int sc, mn;
                    oracle_q4k_scale_min(sb, j, &sc, &mn);
                    int64_t p = 0, sa = 0;
                    for (int i = 32 * j; i < 32 * j + 32; ++i) {
                        const int64_t a = q[m * K + t * 256 + i];
                        p += (int64_t)oracle_q4k_code(sb, i) * a;
                        sa += a;
                    }
                    const float D = d * (float)sc, Mn = dmin * (float)mn;
                    f = fmaf((float)p, D, f);
                    f = fmaf(-(float)sa, Mn, f);
                }
            }
            y[m * N + n] = f * s_a[m];
        }
    }
    return ORACLE_OK;
}

/* W8A8, per-output-channel scale (R3).  acc may be NULL. */
int oracle_gemm_w8a8(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w,
                     float* y, int32_t* acc, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N <= 0 || K <= 0) return ORACLE_ERR_ARG;
    if (M > 0 && (!q || !s_a || !w || !s_w || !y)) return ORACLE_ERR_ARG;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)q[m * K + k] * (int64_t)w[n * K + k];
            if (sum >= INT32_LIMIT || sum < -INT32_LIMIT) {
#pragma omp atomic write
                status = ORACLE_ERR_RANGE;
            }
            int32_t a = (int32_t)sum;
            if (acc) acc[m * N + n] = a;
            float t = (float)a * s_a[m];
            y[m * N + n] = t * s_w[n];
        }
    }
    return status;
}

/* W4A8 with packed signed nibbles (R5) and a per-channel scale (R3). */
int oracle_gemm_w4a8(const int8_t* q, const float* s_a, const uint8_t* w4, const float* s_w,
                     float* y, int32_t* acc, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N <= 0 || K <= 0 || K % 2 != 0) return ORACLE_ERR_ARG;
    if (M > 0 && (!q || !s_a || !w4 || !s_w || !y)) return ORACLE_ERR_ARG;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* wr = w4 + n * (K / 2);
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)q[m * K + k] * (int64_t)oracle_w4_at(wr, k);
            if (sum >= INT32_LIMIT || sum < -INT32_LIMIT) {
#pragma omp atomic write
                status = ORACLE_ERR_RANGE;
            }
            int32_t a = (int32_t)sum;
            if (acc) acc[m * N + n] = a;
            float t = (float)a * s_a[m];
            y[m * N + n] = t * s_w[n];
        }
    }
    return status;
}

/* W8A8 with one fp16 scale per 32 consecutive k of each weight row (R4).
 * d holds the binary16 bit patterns, [N][K/32].  partials may be NULL; if
 * given it receives P[m][n][b], the exact int32 sum of block b. */
int oracle_gemm_w8a8_blockscale(const int8_t* q, const float* s_a, const int8_t* w,
                                const uint16_t* d, float* y, int32_t* partials,
                                int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N <= 0 || K <= 0 || K % 32 != 0) return ORACLE_ERR_ARG;
    if (M > 0 && (!q || !s_a || !w || !d || !y)) return ORACLE_ERR_ARG;
    const int64_t NB = K / 32;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float f = 0.0f;
            for (int64_t b = 0; b < NB; ++b) {
                int64_t sum = 0;
                for (int64_t k = 32 * b; k < 32 * b + 32; ++k)
                    sum += (int64_t)q[m * K + k] * (int64_t)w[n * K + k];
                if (sum >= INT32_LIMIT || sum < -INT32_LIMIT) {
#pragma omp atomic write
                    status = ORACLE_ERR_RANGE;
                }
                int32_t p = (int32_t)sum;
                if (partials) partials[(m * N + n) * NB + b] = p;
                f = fmaf((float)p, oracle_f16_to_f32(d[n * NB + b]), f);
            }
            y[m * N + n] = f * s_a[m];
        }
    }
    return status;
}
