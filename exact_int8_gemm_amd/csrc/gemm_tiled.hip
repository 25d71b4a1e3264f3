// Launchers of the LDS-tiled GEMMs (kernels in gemm_tiled_kernels.h): the
// tile shape is a function of (M, N, K) only.  Every choice computes the same
// exact int32 sums and the same per-element epilogue, so the choice never
// changes a result bit.
#include <atomic>

#include "gemm_pingpong.h"
#include "../../include/prism.h"

namespace prism {
namespace tiled {
namespace dma {

int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;  // MI355X
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace dma
}  // namespace tiled

namespace {

using tiled::launch_tiled;

inline int64_t tiles(int64_t M, int64_t N, int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); }

// 4-bit weights (unpacked on the way into LDS, so a stage costs more and the
// int8 fit below does not carry over): 128 x 128 or 64 x 128 tiles of 8
// waves, two workgroups per CU, K split over s = 1..4 workgroups (each with
// at least 8 stages of 128 k).  Cost model fitted on MI355X (N x K = 12288 x
// 4096 at M = 65..256; 4096 x 4096, 2560 x 9728 and 28672 x 4096 at M = 96
// and 128; 28672 x 14336 at M = 16): per stage of a workgroup alone on its
// CU about 0.72 us for 128 x 128 and 0.53 us for 64 x 128, with two
// workgroups per CU about 0.80 and 0.78 us each (the second one hides part
// of the first one's load latency), times the stages per workgroup and the
// rounds of 512 workgroups; for s > 1 plus the fill, the atomic partial
// tiles and the epilogue kernel, about 5 us and 3 us per split and million
// outputs.  Ties go to 128 x 128 and the smaller split.  E.g. 12288 x 4096:
// M = 128 takes 64 x 128 unsplit (26.3 -> 16.8 us against 128 x 128 split
// in two); M = 96, N = K = 4096: 64 x 128, 4 ways (15.2 -> 13.8 us); M =
// 128, N = 28672: 128 x 128 unsplit (26.7 us against 29.7); M = 16, N x K =
// 28672 x 14336: 64 x 128, 2 ways (61.0 -> 51.3 us).
struct SplitChoice {
  int tile;    // 0: 128 x 128, 1: 64 x 128 (int8 only: 2: 128 x 96)
  int splits;  // 1..4
};

SplitChoice split_int4(int64_t M, int64_t N, int K) {
  const int64_t stages = (K + 127) / 128;
  static constexpr int kBm[2] = {128, 64};
  static constexpr double kAlone[2] = {0.72, 0.53}, kShared[2] = {0.80, 0.78};
  SplitChoice best{0, 1};
  double best_cost = 0.0;
  for (int i = 0; i < 2; ++i) {
    const int64_t t = tiles(M, N, kBm[i], 128);
    for (int s = 1; s <= 4 && (s == 1 || stages / s >= 8); ++s) {
      const int64_t wgs = t * s;
      const double per_stage = wgs <= 256 ? kAlone[i] : kShared[i] * (double)((wgs + 511) / 512);
      double cost = per_stage * (double)((stages + s - 1) / s);
      if (s > 1) cost += 5.0 + 3.0 * (double)s * (double)(M * N) * 1e-6;
      if ((i == 0 && s == 1) || cost < best_cost) {
        best = SplitChoice{i, s};
        best_cost = cost;
      }
    }
  }
  return best;
}

// Tile (128 x 128, 64 x 128 or 128 x 96) and K split s in 1..4 of the int8
// launches with few tiles, from a cost model fitted on MI355X (51 shapes, M
// from 64 to 1024, N and K in {2560, 5120, 9728}, every candidate timed): per
// stage of 128 k, about 0.80 us for 128 x 128 tiles, 0.60 us for 64 x 128
// (both with 8 waves) and 0.78 us for 128 x 96 (4 waves; copies of 32, 24 and
// 28 KiB), times the stages per workgroup and the rounds of up to 256
// workgroups, ceil(tiles s / 256) x ceil(stages / s); plus for s > 1 the fill,
// the in-place epilogue and the atomic partial tiles, about 5 us and 5 us
// per split and million outputs.  128 x 96 tiles pay only up to a 2-way
// split (with 3 or 4 they were 1-4% slower than the other choices).  Ties
// go to the earlier tile and the smaller split.  On the 51 shapes the pick
// was on average 0.2% and at most 5% slower than the best candidate.  E.g.
// M = 512, N = K = 2560: 64 x 128, no split, 11 us (128 x 128: 16 us);
// M = 512, N = K = 5120: 128 x 96, no split, 31 us; M = 512, N = 2560,
// K = 9728: 128 x 128, 3 ways, 36 us.
SplitChoice split_for(int64_t M, int64_t N, int K) {
  struct Shape {
    int bm, bn, max_splits;
    double per_stage;
  };
  // One row of 64 x 128 tiles (M <= 64) shares its few activation rows
  // through L2: about 0.40 us per stage up to 32 rows and 0.50 up to 64 (N
  // from 2560 to 28672; e.g. M = 64, N x K = 16384 x 9728 then splits in two,
  // 42.5 -> 36.5 us).
  const double per_stage_64 = M <= 32 ? 0.40 : M <= 64 ? 0.50 : 0.60;
  const Shape kShapes[3] = {{128, 128, 4, 0.80}, {64, 128, 4, per_stage_64}, {128, 96, 2, 0.78}};
  const int64_t stages = (K + 127) / 128;
  SplitChoice best{0, 1};
  double best_cost = 0.0;
  bool first = true;
  for (int i = 0; i < 3; ++i) {
    const Shape& sh = kShapes[i];
    const int64_t t = tiles(M, N, sh.bm, sh.bn);
    for (int s = 1; s <= sh.max_splits && s <= stages; ++s) {
      const double rounds = (double)((t * s + 255) / 256);
      double cost = sh.per_stage * rounds * (double)((stages + s - 1) / s);
      if (s > 1) cost += 5.0 + 5.0 * (double)s * (double)(M * N) * 1e-6;
      if (first || cost < best_cost) {
        best = SplitChoice{i, s};
        best_cost = cost;
        first = false;
      }
    }
  }
  return best;
}

// int8 weights: direct-to-LDS pipelines (gemm_pingpong.h and
// gemm_tiled_kernels.h, namespace dma).  A launch runs in waves of up to 256
// tiles (one per CU), so its time is about ceil(tiles / 256) times the time
// of one wave of tiles.  Per wave, relative to a 256 x 256 tile (measured on
// MI355X): 256 x 192 0.83 and 256 x 320 1.23 (one-round launches at M = 2048,
// N = K = 5120), 256 x 128 0.60 and 128 x 128 0.45 (M = 8192, three (N, K)
// shapes).  The shape with the smallest estimate wins; ties go to the earlier
// shape in the order 256 x 256, 256 x 320, 256 x 192, 256 x 128, 128 x 128,
// 192 x 128 (0.55: 9-13% faster than 256 x 128 where its tiles fit in one
// round or save one, e.g. M = 512, N = 9728, K = 2560: 28.2 -> 25.6 us):
//  * 256 x 192 / 256 / 320 tiles: 8 waves of 64 x (tile width / 2) in two
//    groups that alternate between MFMAs and LDS reads (gemm_pingpong.h),
//    128-byte stages, 2-deep ring, one persistent workgroup per CU; the
//    320-wide tiles read one 32-k step of fragments per phase (their
//    accumulators take 160 registers);
//  * 192 x 128 tiles: 8 waves of 96 x 32, 3-deep ring;
//  * 256 x 128 tiles: 16 waves of 64 x 32, 3-deep ring (16 waves instead of
//    8: 5-15% faster, e.g. M = 512, N = 9728, K = 2560: 30.6 -> 27.9 us);
//  * 128 x 128 tiles: 8 waves of 32 x 64, 4-deep ring, or, where split_for
//    finds them faster, 64 x 128 tiles of 8 waves of 32 x 32 or 128 x 96
//    tiles of 4 waves of 32 x 96; with K split over up to 4 workgroups per
//    tile (split_for) whose exact int32 partial tiles are added atomically.
//    (8 waves instead of 4 took 2-20% off the 128 x 128 and 64 x 128
//    launches, e.g. M = 512, N = K = 2560 unsplit: 20.4 -> 16.4 us.)
// E.g. M = 8192, N = K = 5120: 640 tiles of 256 x 256 take three rounds for
// 2.5 rounds of work, 512 tiles of 256 x 320 exactly two (272 -> 245 us);
// M = 2048, N = 5120: 216 tiles of 256 x 192 fill the CUs that 160 tiles of
// 256 x 256 leave idle (88 -> 74 us).
void pick_int8(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc, int M,
               int N, int K, hipStream_t st) {
  auto rounds = [](int64_t t) { return (double)((t + 255) / 256); };
  const double cost[6] = {rounds(tiles(M, N, 256, 256)),        1.23 * rounds(tiles(M, N, 256, 320)),
                          0.83 * rounds(tiles(M, N, 256, 192)), 0.60 * rounds(tiles(M, N, 256, 128)),
                          0.45 * rounds(tiles(M, N, 128, 128)), 0.55 * rounds(tiles(M, N, 192, 128))};
  int best = 0;
  for (int i = 1; i < 6; ++i)
    if (cost[i] < cost[best]) best = i;
  switch (best) {
    case 0: tiled::dma::launch_pp<128>(q, s_a, w, s_w, y, acc, M, N, K, st); break;
    case 1: tiled::dma::launch_pp<128, 320, 1>(q, s_a, w, s_w, y, acc, M, N, K, st); break;
    case 2: tiled::dma::launch_pp<128, 192>(q, s_a, w, s_w, y, acc, M, N, K, st); break;
    case 3: tiled::dma::launch<256, 128, 128, 4, 4, 3, 1>(q, s_a, w, s_w, y, acc, M, N, K, st); break;
    case 5: tiled::dma::launch<192, 128, 128, 2, 4, 3, 1>(q, s_a, w, s_w, y, acc, M, N, K, st); break;
    default: {
      const SplitChoice c = split_for(M, N, K);
      if (c.tile == 1) tiled::dma::launch<64, 128, 128, 2, 4, 4, 1>(q, s_a, w, s_w, y, acc, M, N, K, st, c.splits);
      else if (c.tile == 2) tiled::dma::launch<128, 96, 128, 4, 1, 4, 1>(q, s_a, w, s_w, y, acc, M, N, K, st, c.splits);
      else tiled::dma::launch<128, 128, 128, 4, 2, 4, 1>(q, s_a, w, s_w, y, acc, M, N, K, st, c.splits);
    }
  }
}

// 4-bit weights, two kernels:
//  * the persistent ping-pong kernel on 256-row tiles with the packed bytes
//    copied to LDS as they are (256 x 192, 256 x 256 or 256 x 320);
//  * a register-staged pipeline that unpacks the nibbles on their way into
//    LDS: 128 x 128 tiles of 8 waves (32 x 64 each; 4-20% faster than 4 waves
//    of 64 x 64, e.g. M = 256, N = K = 5120: 38.5 -> 30.3 us) or 64 x 128
//    tiles of 8 waves (32 x 32 each; 8 waves of 64 x 32 took 20-21 against
//    17 us at M = 65..128 on 12288 x 4096), two workgroups per CU, tile and
//    K split from split_int4.
// Estimates in us per 1024 of K, fitted on MI355X with weights that do not
// stay in cache (N x K = 12288 x 4096, 9728 x 2560, 2560 x 9728, 5120 x 5120
// and 17408 x 5120, M = 96..2048): 11.7 per 256-tile round of 256 x 192
// (14.1 and 17.3 for 256 x 256 and 256 x 320, the int8 ratios, which this
// sweep does not separate).  128 x 128 always wins while its t tiles fit the
// 512 workgroups that run together (two per CU); past that it takes about
// 0.02 t + 3, the remainder adding a second, partly filled wave.  Against the
// earlier rule (0.63 per 512 tiles of 128 x 128, at least 0.63) this moves
// 17 shapes from 128 x 128 to 256-row tiles, bits unchanged: M x N x K =
// 512 x 17408 x 5120: 78.5 -> 68.4 us, 768 x 12288 x 4096: 60.8 -> 54.1,
// 1024 x 9728 x 2560: 43.1 -> 38.4, 2048 x 5120 x 5120: 77.4 -> 66.8,
// 4096 x 2560 x 9728: 133.6 -> 114.8, 6144 x 4096 x 14336: 393 -> 336
// (2331 -> 2091 us summed over the 17 and the four it leaves at exactly 512
// tiles).
void pick_int4(const int8_t* q, const float* s_a, const int8_t* w, const float* s_w, float* y, int32_t* acc, int M,
               int N, int K, hipStream_t st) {
  auto rounds = [](int64_t t) { return (double)((t + 255) / 256); };
  const double pp[3] = {11.7 * rounds(tiles(M, N, 256, 192)), 14.1 * rounds(tiles(M, N, 256, 256)),
                        17.3 * rounds(tiles(M, N, 256, 320))};
  const int64_t t128 = tiles(M, N, 128, 128);
  const double c128 = t128 <= 512 ? 0.0 : 0.02 * (double)t128 + 3.0;
  int best = 0;
  for (int i = 1; i < 3; ++i)
    if (pp[i] < pp[best]) best = i;
  if (pp[best] < c128) {
    if (best == 0) tiled::dma::launch_pp<128, 192, 2, true>(q, s_a, w, s_w, y, acc, M, N, K, st);
    else if (best == 1) tiled::dma::launch_pp<128, 256, 2, true>(q, s_a, w, s_w, y, acc, M, N, K, st);
    else tiled::dma::launch_pp<128, 320, 1, true>(q, s_a, w, s_w, y, acc, M, N, K, st);
    return;
  }
  const SplitChoice c = split_int4(M, N, K);
  if (c.tile == 1) launch_tiled<64, 128, 128, 2, 4, true, 2>(q, s_a, w, s_w, y, acc, M, N, K, st, c.splits);
  else launch_tiled<128, 128, 128, 4, 2, true, 2>(q, s_a, w, s_w, y, acc, M, N, K, st, c.splits);
}

}  // namespace

// One named entry of the table above (7: 256 x 256, 8: 256 x 128, 9..12:
// 128 x 128 with K split over 1..4 workgroups, 17: 256 x 192, 18: 256 x 320,
// 19..22: 64 x 128 with K split over 1..4 workgroups, 23, 24: 128 x 96 with
// K split over 1, 2 workgroups, 26: 192 x 128; the 4-bit path has 7, 9..12,
// 17, 18 and 19..22).
int launch_gemm_tiled_variant(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w,
                              float* y, int32_t* acc, int M, int N, int K, int variant, hipStream_t st) {
  const int8_t* wb = static_cast<const int8_t*>(w);
  if (w_is_int4) {
    if (variant == 7 || variant == 17 || variant == 18) {
      if (variant == 7) tiled::dma::launch_pp<128, 256, 2, true>(q, s_a, wb, s_w, y, acc, M, N, K, st);
      else if (variant == 17) tiled::dma::launch_pp<128, 192, 2, true>(q, s_a, wb, s_w, y, acc, M, N, K, st);
      else tiled::dma::launch_pp<128, 320, 1, true>(q, s_a, wb, s_w, y, acc, M, N, K, st);
      return launch_status();
    }
    const bool t64 = variant >= 19 && variant <= 22;
    if (!t64 && (variant < 9 || variant > 12)) return PRISM_ERR_INVALID_ARG;  // 128 x 128 or 64 x 128 only
    const int stages = (K + 127) / 128;
    int splits = t64 ? variant - 18 : variant - 8;
    if (splits > stages) splits = stages;
    if (t64) launch_tiled<64, 128, 128, 2, 4, true, 2>(q, s_a, wb, s_w, y, acc, M, N, K, st, splits);
    else launch_tiled<128, 128, 128, 4, 2, true, 2>(q, s_a, wb, s_w, y, acc, M, N, K, st, splits);
    return launch_status();
  }
  if (variant == 7) {
    tiled::dma::launch_pp<128>(q, s_a, wb, s_w, y, acc, M, N, K, st);
  } else if (variant == 17) {
    tiled::dma::launch_pp<128, 192>(q, s_a, wb, s_w, y, acc, M, N, K, st);
  } else if (variant == 18) {
    tiled::dma::launch_pp<128, 320, 1>(q, s_a, wb, s_w, y, acc, M, N, K, st);
  } else if (variant == 8) {
    tiled::dma::launch<256, 128, 128, 4, 4, 3, 1>(q, s_a, wb, s_w, y, acc, M, N, K, st);
  } else if (variant >= 9 && variant <= 12) {
    const int stages = (K + 127) / 128;
    int splits = variant - 8;
    if (splits > stages) splits = stages;
    tiled::dma::launch<128, 128, 128, 4, 2, 4, 1>(q, s_a, wb, s_w, y, acc, M, N, K, st, splits);
  } else if (variant >= 19 && variant <= 22) {
    const int stages = (K + 127) / 128;
    int splits = variant - 18;
    if (splits > stages) splits = stages;
    tiled::dma::launch<64, 128, 128, 2, 4, 4, 1>(q, s_a, wb, s_w, y, acc, M, N, K, st, splits);
  } else if (variant == 26) {
    tiled::dma::launch<192, 128, 128, 2, 4, 3, 1>(q, s_a, wb, s_w, y, acc, M, N, K, st);
  } else if (variant == 23 || variant == 24) {
    const int stages = (K + 127) / 128;
    int splits = variant - 22;
    if (splits > stages) splits = stages;
    tiled::dma::launch<128, 96, 128, 4, 1, 4, 1>(q, s_a, wb, s_w, y, acc, M, N, K, st, splits);
  } else {
    return PRISM_ERR_INVALID_ARG;
  }
  return launch_status();
}

int launch_gemm_tiled(const int8_t* q, const float* s_a, const void* w, bool w_is_int4, const float* s_w, float* y,
                      int32_t* acc, int M, int N, int K, hipStream_t st) {
  const int8_t* wb = static_cast<const int8_t*>(w);
  if (w_is_int4) pick_int4(q, s_a, wb, s_w, y, acc, M, N, K, st);
  else pick_int8(q, s_a, wb, s_w, y, acc, M, N, K, st);
  return launch_status();
}

// Block scales: direct-to-LDS pipeline with the scales riding along in each
// stage; 128 x 64 tiles of 4 waves, three workgroups per CU (the fp32 block
// combine is VALU-bound: the other workgroups keep the VALU busy while one
// waits; at M = 2048, N = 17408, K = 5120 this beat 128 x 128 tiles at two
// workgroups per CU by about 15%).
int launch_gemm_blockscale(const int8_t* q, const float* s_a, const int8_t* w, const uint16_t* d, float* y,
                           int32_t* partials, int M, int N, int K, hipStream_t st) {
  if (M <= kBlockSmallMMax && !partials)
    return launch_gemm_block_small(q, s_a, w, d, nullptr, y, M, N, K, st);
  // 128 x 128 tiles of eight waves (two workgroups per CU) from four rounds of
  // the CUs' workgroup slots up, else 128 x 64 tiles of four waves (three per
  // CU).  MI355X, 17408 x 5120: M = 2048 430 -> 410 us, M = 4096 825 -> 791
  // us; at M = 512 the larger tiles took 145 against 120-126 us.  The variant
  // that also stores every block sum keeps the smaller tiles (the larger
  // ones would spill it).
  // Up to 64 rows, 64 x 64 tiles of four waves (four workgroups per CU): the
  // fold then runs on at most 63 rows past M instead of 111 (M = 17: 46 -> 41
  // us, M = 64: 51 -> 47 us; from M = 96 on they are slower).
  const int64_t tiles128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  if (M <= 64)
    tiled::dma::launch_block<64, 64, 2, 2, 2, 4>(q, s_a, w, d, y, partials, M, N, K, st);
  else if (!partials && tiles128 >= 4 * 2 * (int64_t)tiled::dma::device_cus())
    tiled::dma::launch_block<128, 128, 4, 2, 2, 2, false>(q, s_a, w, d, y, nullptr, M, N, K, st);
  else
    tiled::dma::launch_block<128, 64, 2, 2, 2, 3>(q, s_a, w, d, y, partials, M, N, K, st);
  return launch_status();
}

// Q4_K-native W4A8 on the repacked planes (packed codes and super-block
// headers): the block-scale pipeline with the scales decoded from the headers
// (128 x 128 tiles, two workgroups per CU).
int launch_gemm_q4k(const int8_t* q, const float* s_a, const uint8_t* w4, const uint8_t* hdr, float* y, int M, int N,
                    int K, hipStream_t st) {
  if (M <= kBlockSmallMMax)
    return launch_gemm_block_small(q, s_a, reinterpret_cast<const int8_t*>(w4), nullptr, hdr, y, M, N, K, st);
  // 128 x 128 tiles of eight waves (32 x 64 each, two workgroups per CU) when
  // they fill at least two rounds of the CUs' workgroup slots, else 64 x 64
  // tiles of four waves (four workgroups per CU): few rows then waste less of
  // the per-block fold on rows past M, and the more numerous tiles fill the
  // CUs.  MI355X, 17408 x 5120, against 128 x 128 tiles of four waves: M = 17
  // 80 -> 47 us, 128 83 -> 64, 256 109 -> 98, 512 220 -> 172, 1024 339 ->
  // 313, 2048 589 -> 561, 4096 1109 -> 1086.
  const int64_t tiles128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  if (tiles128 >= 2 * 2 * (int64_t)tiled::dma::device_cus())
    tiled::dma::launch_q4k<128, 128, 4, 2, 2, 2>(q, s_a, w4, hdr, y, M, N, K, st);
  else
    tiled::dma::launch_q4k<64, 64, 2, 2, 2, 4>(q, s_a, w4, hdr, y, M, N, K, st);
  return launch_status();
}

}  // namespace prism
