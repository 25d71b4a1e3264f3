// C ABI of libprism: argument validation, device check and shape dispatch.
//
// Every call validates its arguments before touching HIP, so an invalid
// call enqueues nothing and writes nothing (the pages' servers refuse
// oversized requests instead of truncating them; this library does the same
// with unsupported shapes).  The kernel choice depends on (M, N, K) only and
// never changes a result bit: sums are exact in int32 and each epilogue is a
// fixed per-element sequence of fp32 operations.
#include <atomic>
#include <climits>
#include <cstring>

#include <hip/hip_runtime.h>

#include "../../include/prism.h"
#include "prism_internal.h"

#ifndef PRISM_BUILD_ID
#error "PRISM_BUILD_ID (the source hash written by build.py) must be defined"
#endif

namespace prism {

int launch_status() { return hipGetLastError() == hipSuccess ? PRISM_OK : PRISM_ERR_LAUNCH; }

}  // namespace prism

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

// Also clears an error that an earlier, unrelated HIP call left on this thread,
// so that launch_status() after this call's launches reports those launches only.
int check_device() {
  (void)hipGetLastError();
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return PRISM_ERR_UNSUPPORTED;
  if (dev < kMaxDevices) {
    const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return PRISM_OK;
    if (c == 2) return PRISM_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PRISM_ERR_UNSUPPORTED;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                  (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? PRISM_OK : PRISM_ERR_UNSUPPORTED;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shared checks of the three GEMM calls.  Returns PRISM_OK to go on, or a
// status; *noop is set when M == 0.
int check_gemm(const void* q, const void* s_a, const void* w, const void* scale_w, const void* y,
               const void* acc_or_partials, int64_t M, int64_t N, int64_t K, int k_multiple, bool* noop) {
  *noop = false;
  if (M < 0 || N < 0 || K < 0) return PRISM_ERR_INVALID_ARG;
  if (M == 0) {
    *noop = true;
    return PRISM_OK;
  }
  if (N == 0 || K == 0 || K > PRISM_K_MAX || M > INT_MAX || N > INT_MAX) return PRISM_ERR_INVALID_ARG;
  if (!q || !s_a || !w || !scale_w || !y) return PRISM_ERR_INVALID_ARG;
  if (K % k_multiple != 0) return PRISM_ERR_ALIGNMENT;
  if (!aligned(q, 16) || !aligned(w, 16) || !aligned(s_a, 4) || !aligned(y, 4) || !aligned(acc_or_partials, 4))
    return PRISM_ERR_ALIGNMENT;
  return PRISM_OK;
}

// Grid limits of the tiled kernels (64 x 128 tiles with a 4-way K split at the most).
bool grid_fits(int64_t M, int64_t N) { return ((M + 63) / 64) * ((N + 127) / 128) * 4 <= INT_MAX; }

// The small-M kernel re-reads the whole M x K activation block in every
// workgroup, so from some rows on the 64 x 128 tiles of the tiled path (K
// split by their cost model) are faster.  Where, measured on MI355X with
// graph-replayed launches and the weights rotated through at least 640 MB
// (so that they come from HBM, as in a model's forward pass), M = 8, 16,
// 24, 32, 48, 64; N in {2560, 5120, 9728, 12288, 16384, 18432, 28672}; K in
// {2560, 4096, 5120, 9728, 14336}:
//  * N > 16384 (no even column share per CU fits the small-M kernel, whose
//    16-column blocks then run in several rounds): from 8 int8 rows (18432
//    x 5120, M = 16: 30.3 -> 28.8 us; 28672 x 2560, M = 64: 56.9 -> 20.4
//    us); 4-bit from 24 rows, or 16 where K >= 8192 (28672 x 4096, M = 48:
//    34.3 -> 22.9 us; 18432 x 4096, M = 16 stays: 14.8 against 18.2 us);
//  * int8 weights up to 16384 columns: from 24 rows where M K >= 229376
//    (5120 x 9728, M = 24: 20.6 -> 19.1 us; 9728 x 14336, M = 24: 38.3 ->
//    34.3 us; 5120 x 2560, M = 64 stays: 12.1 against 13.9 us);
//  * 4-bit weights up to 16384 columns: from 48 rows where M K >= 393216
//    and from 32 rows where N K >= 128 Mi (5120 x 9728, M = 48: 24.0 ->
//    18.5 us; 16384 x 14336, M = 32: 41.2 -> 35.1 us).
// Over those 210 shapes the calls take 5541 against 6125 us (int8) and 4221
// against 4808 us (4-bit) with the rule of small-M up to 64 rows except
// int8 from 32 rows and M K >= 245760; the int8 part was then narrowed where
// small-M stayed faster (12288 x 4096 and 16384 x 2560 at M = 24, 32).
bool use_small(int64_t M, int64_t N, int64_t K, bool w4) {
  if (M > prism::kSmallMMax) return false;
  if (w4) {
    if (N > 16384) return !(M >= 24 || (M >= 16 && K >= 8192));
    return !((M >= 48 && M * K >= 393216) || (M >= 32 && N * K >= (int64_t)128 << 20));
  }
  if (N > 16384) return M < 8;
  return !(M >= 24 && M * K >= 229376);
}

// Variant dispatch shared by the two _variant calls (arguments already checked).
int run_variant(const int8_t* q, const float* s_a, const void* w, bool w4, const float* s_w, float* y, int32_t* acc,
                int64_t M, int64_t N, int64_t K, int variant, hipStream_t s) {
  static const int kSmall[7][2] = {{0, 0}, {1, 4}, {1, 8}, {1, 16}, {2, 4}, {2, 8}, {2, 16}};
  static const int kSmallWide[4][2] = {{3, 4}, {3, 8}, {4, 4}, {4, 8}};
  if (variant == PRISM_VARIANT_AUTO) {
    if (use_small(M, N, K, w4)) return prism::launch_gemm_small(q, s_a, w, w4, s_w, y, acc, (int)M, (int)N, (int)K, s);
    return prism::launch_gemm_tiled(q, s_a, w, w4, s_w, y, acc, (int)M, (int)N, (int)K, s);
  }
  if (variant >= PRISM_VARIANT_SMALL_1x4 && variant <= PRISM_VARIANT_SMALL_2x16) {
    if (M > prism::kSmallMMax) return PRISM_ERR_INVALID_ARG;
    return prism::launch_gemm_small_variant(q, s_a, w, w4, s_w, y, acc, (int)M, (int)N, (int)K, kSmall[variant][0],
                                            kSmall[variant][1], s);
  }
  if (variant >= PRISM_VARIANT_SMALL_3x4 && variant <= PRISM_VARIANT_SMALL_4x8) {
    if (M > prism::kSmallMMax) return PRISM_ERR_INVALID_ARG;
    const int* e = kSmallWide[variant - PRISM_VARIANT_SMALL_3x4];
    return prism::launch_gemm_small_variant(q, s_a, w, w4, s_w, y, acc, (int)M, (int)N, (int)K, e[0], e[1], s);
  }
  if (variant == PRISM_VARIANT_SMALL_BALANCED) {
    if (M > prism::kSmallMMax) return PRISM_ERR_INVALID_ARG;
    return prism::launch_gemm_small_balanced(q, s_a, w, w4, s_w, y, acc, (int)M, (int)N, (int)K, s);
  }
  if ((variant >= PRISM_VARIANT_TILE_256x256 && variant <= PRISM_VARIANT_TILE_128x128_SPLIT4) ||
      (variant >= PRISM_VARIANT_TILE_256x192 && variant <= PRISM_VARIANT_TILE_128x96_SPLIT2) ||
      variant == PRISM_VARIANT_TILE_192x128)
    return prism::launch_gemm_tiled_variant(q, s_a, w, w4, s_w, y, acc, (int)M, (int)N, (int)K, variant, s);
  return PRISM_ERR_INVALID_ARG;
}


}  // namespace

extern "C" {

int prism_abi_version(void) { return PRISM_ABI_VERSION; }

const char* prism_build_id(void) { return PRISM_BUILD_ID; }

const char* prism_status_string(int status) {
  switch (status) {
    case PRISM_OK: return "ok";
    case PRISM_ERR_INVALID_ARG: return "invalid argument (null pointer, negative or zero size, or K above PRISM_K_MAX)";
    case PRISM_ERR_ALIGNMENT: return "misaligned pointer or K not a multiple of the required block";
    case PRISM_ERR_UNSUPPORTED: return "no usable gfx950 (MI355X) device is current";
    case PRISM_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int prism_quantize_rows(const float* x, int8_t* q, float* scale, int64_t M, int64_t K, void* stream) {
  if (M < 0 || K < 0) return PRISM_ERR_INVALID_ARG;
  if (M == 0) return PRISM_OK;
  if (K == 0 || M > INT_MAX || K > INT_MAX / 4) return PRISM_ERR_INVALID_ARG;
  if (!x || !q || !scale) return PRISM_ERR_INVALID_ARG;
  if (K % 16 != 0 || !aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return PRISM_ERR_ALIGNMENT;
  const int dev = check_device();
  if (dev != PRISM_OK) return dev;
  return prism::launch_quantize_rows(x, q, scale, M, K, static_cast<hipStream_t>(stream));
}

int prism_quantize_rows_static(const float* x, int8_t* q, float* scale, float s, int64_t M, int64_t K,
                               void* stream) {
  if (M < 0 || K < 0) return PRISM_ERR_INVALID_ARG;
  if (!(s > 0.0f) || s == __builtin_inff()) return PRISM_ERR_INVALID_ARG;  // NaN, zero, negative, +inf
  if (M == 0) return PRISM_OK;
  if (K == 0 || M > INT_MAX || K > INT_MAX / 4) return PRISM_ERR_INVALID_ARG;
  if (!x || !q || !scale) return PRISM_ERR_INVALID_ARG;
  if (K % 16 != 0 || !aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return PRISM_ERR_ALIGNMENT;
  const int dev = check_device();
  if (dev != PRISM_OK) return dev;
  return prism::launch_quantize_rows_static(x, q, scale, s, M, K, static_cast<hipStream_t>(stream));
}

int prism_repack_q4_k(const uint8_t* blocks, uint8_t* w4, uint8_t* hdr, int64_t N, int64_t K, void* stream) {
  if (N < 0 || K < 0) return PRISM_ERR_INVALID_ARG;
  if (N == 0) return PRISM_OK;
  if (K == 0 || N > INT_MAX || K > INT_MAX) return PRISM_ERR_INVALID_ARG;
  if (!blocks || !w4 || !hdr) return PRISM_ERR_INVALID_ARG;
  if (K % 256 != 0 || !aligned(blocks, 16) || !aligned(w4, 16) || !aligned(hdr, 16)) return PRISM_ERR_ALIGNMENT;
  if ((N * (K / 256) * 9 + 255) / 256 > INT_MAX) return PRISM_ERR_INVALID_ARG;  // grid size
  const int dev = check_device();
  if (dev != PRISM_OK) return dev;
  return prism::launch_repack_q4_k(blocks, w4, hdr, N, K, static_cast<hipStream_t>(stream));
}

int prism_gemm_w4a8_q4k(const int8_t* q, const float* s_a, const uint8_t* w4, const uint8_t* hdr, float* y, int64_t M,
                        int64_t N, int64_t K, void* stream) {
  bool noop;
  int st = check_gemm(q, s_a, w4, hdr, y, nullptr, M, N, K, 256, &noop);
  if (st != PRISM_OK || noop) return st;
  if (!aligned(hdr, 16)) return PRISM_ERR_ALIGNMENT;
  if (!grid_fits(M, N)) return PRISM_ERR_INVALID_ARG;
  if ((st = check_device()) != PRISM_OK) return st;
  return prism::launch_gemm_q4k(q, s_a, w4, hdr, y, (int)M, (int)N, (int)K, static_cast<hipStream_t>(stream));
}

int prism_repack_q8_0(const uint8_t* blocks, int8_t* w, uint16_t* d, int64_t N, int64_t K, void* stream) {
  if (N < 0 || K < 0) return PRISM_ERR_INVALID_ARG;
  if (N == 0) return PRISM_OK;
  if (K == 0 || N > INT_MAX || K > INT_MAX) return PRISM_ERR_INVALID_ARG;
  if (!blocks || !w || !d) return PRISM_ERR_INVALID_ARG;
  if (K % 32 != 0 || !aligned(blocks, 16) || !aligned(w, 16) || !aligned(d, 2)) return PRISM_ERR_ALIGNMENT;
  if ((N * (K / 32) + 255) / 256 > INT_MAX) return PRISM_ERR_INVALID_ARG;  // grid size
  const int dev = check_device();
  if (dev != PRISM_OK) return dev;
  return prism::launch_repack_q8_0(blocks, w, d, N, K, static_cast<hipStream_t>(stream));
}

int prism_gemm_w8a8(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc,
                    int64_t M, int64_t N, int64_t K, void* stream) {
  bool noop;
  int st = check_gemm(q, s_a, w, s_w, y, acc, M, N, K, 16, &noop);
  if (st != PRISM_OK || noop) return st;
  if (!aligned(s_w, 4)) return PRISM_ERR_ALIGNMENT;
  if (!grid_fits(M, N)) return PRISM_ERR_INVALID_ARG;
  if ((st = check_device()) != PRISM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_small(M, N, K, false))
    return prism::launch_gemm_small(q, s_a, w, false, s_w, y, acc, (int)M, (int)N, (int)K, s);
  return prism::launch_gemm_tiled(q, s_a, w, false, s_w, y, acc, (int)M, (int)N, (int)K, s);
}

int prism_quantize_gemm_w8a8(const float* x, int8_t* q, float* scale, const int8_t* w, const float* s_w, float* y,
                             int32_t* acc, int64_t M, int64_t N, int64_t K, void* stream) {
  bool noop;
  int st = check_gemm(q, scale, w, s_w, y, acc, M, N, K, 16, &noop);
  if (st != PRISM_OK || noop) return st;
  if (!x) return PRISM_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(s_w, 4)) return PRISM_ERR_ALIGNMENT;
  if (!grid_fits(M, N)) return PRISM_ERR_INVALID_ARG;
  if ((st = check_device()) != PRISM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 1 && prism::launch_quantize_gemv(x, q, scale, w, s_w, y, acc, (int)N, (int)K, s))
    return prism::launch_status();
  if (M <= prism::kFusedSmallMMax &&
      prism::launch_quantize_gemm_small(x, q, scale, w, s_w, y, acc, (int)M, (int)N, (int)K, s))
    return prism::launch_status();
  if ((st = prism::launch_quantize_rows(x, q, scale, M, K, s)) != PRISM_OK) return st;
  if (use_small(M, N, K, false))
    return prism::launch_gemm_small(q, scale, w, false, s_w, y, acc, (int)M, (int)N, (int)K, s);
  return prism::launch_gemm_tiled(q, scale, w, false, s_w, y, acc, (int)M, (int)N, (int)K, s);
}

int prism_gemm_w4a8(const int8_t* q, const float* s_a, const uint8_t* w4, const float* s_w, float* y, int32_t* acc,
                    int64_t M, int64_t N, int64_t K, void* stream) {
  bool noop;
  int st = check_gemm(q, s_a, w4, s_w, y, acc, M, N, K, 32, &noop);
  if (st != PRISM_OK || noop) return st;
  if (!aligned(s_w, 4)) return PRISM_ERR_ALIGNMENT;
  if (!grid_fits(M, N)) return PRISM_ERR_INVALID_ARG;
  if ((st = check_device()) != PRISM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_small(M, N, K, true)) return prism::launch_gemm_small(q, s_a, w4, true, s_w, y, acc, (int)M, (int)N, (int)K, s);
  return prism::launch_gemm_tiled(q, s_a, w4, true, s_w, y, acc, (int)M, (int)N, (int)K, s);
}

int prism_gemm_w8a8_variant(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y,
                            int32_t* acc, int64_t M, int64_t N, int64_t K, int variant, void* stream) {
  if (variant < 0 || variant >= PRISM_VARIANT_COUNT) return PRISM_ERR_INVALID_ARG;
  bool noop;
  int st = check_gemm(q, s_a, w, s_w, y, acc, M, N, K, 16, &noop);
  if (st != PRISM_OK || noop) return st;
  if (!aligned(s_w, 4)) return PRISM_ERR_ALIGNMENT;
  if (!grid_fits(M, N)) return PRISM_ERR_INVALID_ARG;
  if ((st = check_device()) != PRISM_OK) return st;
  return run_variant(q, s_a, w, false, s_w, y, acc, M, N, K, variant, static_cast<hipStream_t>(stream));
}

int prism_gemm_w4a8_variant(const int8_t* q, const float* s_a, const uint8_t* w4, const float* s_w, float* y,
                            int32_t* acc, int64_t M, int64_t N, int64_t K, int variant, void* stream) {
  if (variant < 0 || variant >= PRISM_VARIANT_COUNT) return PRISM_ERR_INVALID_ARG;
  bool noop;
  int st = check_gemm(q, s_a, w4, s_w, y, acc, M, N, K, 32, &noop);
  if (st != PRISM_OK || noop) return st;
  if (!aligned(s_w, 4)) return PRISM_ERR_ALIGNMENT;
  if (!grid_fits(M, N)) return PRISM_ERR_INVALID_ARG;
  if ((st = check_device()) != PRISM_OK) return st;
  return run_variant(q, s_a, w4, true, s_w, y, acc, M, N, K, variant, static_cast<hipStream_t>(stream));
}

int prism_gemm_w8a8_blockscale(const int8_t* q, const float* s_a, const int8_t* w, const uint16_t* d, float* y,
                               int32_t* partials, int64_t M, int64_t N, int64_t K, void* stream) {
  bool noop;
  int st = check_gemm(q, s_a, w, d, y, partials, M, N, K, 32, &noop);
  if (st != PRISM_OK || noop) return st;
  if (!aligned(d, 2)) return PRISM_ERR_ALIGNMENT;
  if (!grid_fits(M, N)) return PRISM_ERR_INVALID_ARG;
  if ((st = check_device()) != PRISM_OK) return st;
  return prism::launch_gemm_blockscale(q, s_a, w, d, y, partials, (int)M, (int)N, (int)K,
                                       static_cast<hipStream_t>(stream));
}

int prism_peak_mfma(int64_t iters, int waves_per_simd, int seed, uint32_t* out, void* stream) {
  if (iters < 1 || iters > (1 << 24) || seed < 0 || seed > (1 << 20) || !out) return PRISM_ERR_INVALID_ARG;
  if (waves_per_simd != 1 && waves_per_simd != 2 && waves_per_simd != 4) return PRISM_ERR_INVALID_ARG;
  if (!aligned(out, 4)) return PRISM_ERR_ALIGNMENT;
  int st = check_device();
  if (st != PRISM_OK) return st;
  return prism::launch_peak_mfma(iters, waves_per_simd, seed, out, static_cast<hipStream_t>(stream));
}

int prism_peak_read(const void* buf, int64_t bytes, uint32_t* parts, void* stream) {
  if (!buf || !parts || bytes <= 0 || bytes > ((int64_t)1 << 40)) return PRISM_ERR_INVALID_ARG;
  if (bytes % 16 != 0 || !aligned(buf, 16) || !aligned(parts, 4)) return PRISM_ERR_ALIGNMENT;
  int st = check_device();
  if (st != PRISM_OK) return st;
  return prism::launch_peak_read(buf, bytes, parts, PRISM_PEAK_READ_PARTS, static_cast<hipStream_t>(stream));
}

int prism_peak_fold(int mode, int64_t iters, float* out, void* stream) {
  if (mode < 0 || mode > 4 || iters < 1 || iters > (1 << 20) || !out) return PRISM_ERR_INVALID_ARG;
  if (!aligned(out, 4)) return PRISM_ERR_ALIGNMENT;
  int st = check_device();
  if (st != PRISM_OK) return st;
  return prism::launch_peak_fold(mode, iters, out, static_cast<hipStream_t>(stream));
}

}  // extern "C"
