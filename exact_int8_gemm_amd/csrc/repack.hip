// Q8_0 weight blocks -> the two planes the block-scale GEMM reads.
//
// The pages say that Q8_0 files run as int8 (W8A8) with no conversion step
// (StartLux-Prism README, "Why StartLux-Prism", bullet on the released
// files).  A Q8_0 block (public GGUF layout) is 34 bytes: a little-endian
// binary16 scale, then the 32 int8 codes of 32 consecutive k of one weight
// row; blocks follow each other row by row.  Its values are scale * code,
// which is exactly the (w, d) operand pair of prism_gemm_w8a8_blockscale, so
// this pass only moves bytes: the codes to w [N][K], the scale bits to
// d [N][K/32].  Nothing is converted or rounded.
//
// One workgroup moves 256 blocks (8704 bytes = 544 x 16 bytes): it copies
// them into LDS with 16-byte loads (a buffer resource per workgroup bounds
// every access to the caller's data; a tail that is not a whole number of
// 16-byte pieces is read bytewise, so no byte past the end is touched).
// Then thread t writes the 16-byte halves t and t + 256 of the chunk's 8192
// code bytes, so each store instruction covers 1 KB of w contiguously, and
// threads below 128 write two scales as one dword.  Block i starts at LDS
// byte 34 i, so the codes of every other block start 2 bytes into a dword;
// v_alignbyte_b32 rebuilds them.
#include "prism_internal.h"
#include "../../include/prism.h"

namespace prism {
namespace {

constexpr int kBlockBytes = 34;
constexpr int kPerGroup = 256;
constexpr int kChunkDwords = kPerGroup * kBlockBytes / 4;  // 2176

__global__ __launch_bounds__(kPerGroup) void repack_q8_0_kernel(const uint8_t* __restrict__ blocks,
                                                                 int8_t* __restrict__ w, uint16_t* __restrict__ d,
                                                                 int64_t nblocks) {
  __shared__ uint32_t buf[kChunkDwords + 4];
  const int64_t g0 = (int64_t)blockIdx.x * kPerGroup;
  const int nb = nblocks - g0 < kPerGroup ? (int)(nblocks - g0) : kPerGroup;
  const uint32_t nbytes = (uint32_t)nb * kBlockBytes;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blocks + g0 * kBlockBytes), (short)0, (int)nbytes,
                                        0x00020000);
  const uint32_t nfull = nbytes / 16;  // whole 16-byte pieces
  for (uint32_t i = threadIdx.x; i < nfull; i += kPerGroup) {
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, i * 16, 0, 0);
    buf[4 * i] = (uint32_t)v[0];
    buf[4 * i + 1] = (uint32_t)v[1];
    buf[4 * i + 2] = (uint32_t)v[2];
    buf[4 * i + 3] = (uint32_t)v[3];
  }
  // Tail bytes (fewer than 16), one dword per thread, bytewise.
  const uint32_t tail0 = nfull * 4, ndw = (nbytes + 3) / 4;
  for (uint32_t i = tail0 + threadIdx.x; i < ndw; i += kPerGroup) {
    uint32_t v = 0;
    for (uint32_t b = 0; b < 4 && i * 4 + b < nbytes; ++b)
      v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, i * 4 + b, 0, 0) << (8 * b);
    buf[i] = v;
  }
  __syncthreads();

  // Codes: piece h (0 .. 2 nb - 1) is bytes 16 (h % 2) .. + 15 of the codes of block h / 2.
  int8_t* wg = w + g0 * 32;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int h = threadIdx.x + pass * kPerGroup;
    if (h < 2 * nb) {
      const uint32_t c0 = (uint32_t)(h >> 1) * kBlockBytes + 2 + 16 * (h & 1), j = c0 >> 2;
      const bool shifted = (c0 & 3) != 0;  // the piece starts 2 bytes into dword j
      uint32_t c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        c[i] = shifted ? __builtin_amdgcn_alignbyte(buf[j + i + 1], buf[j + i], 2) : buf[j + i];
      *reinterpret_cast<v4i*>(wg + (int64_t)h * 16) = v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
    }
  }
  // Scales: thread t < 128 writes those of blocks 2t and 2t + 1 (one dword; d is
  // 2-byte aligned only, so an odd-address d takes two 2-byte stores).
  const int t = threadIdx.x;
  if (2 * t < nb) {
    auto scale_of = [&](int i) -> uint32_t {
      const uint32_t o = (uint32_t)i * kBlockBytes;  // o % 4 is 0 or 2: the scale sits inside one dword
      return (buf[o >> 2] >> ((o & 3) * 8)) & 0xffffu;
    };
    const int64_t g = g0 + 2 * t;
    const uint32_t s0 = scale_of(2 * t);
    if (2 * t + 1 < nb && ((reinterpret_cast<uintptr_t>(d + g) & 3) == 0)) {
      *reinterpret_cast<uint32_t*>(d + g) = s0 | (scale_of(2 * t + 1) << 16);
    } else {
      d[g] = (uint16_t)s0;
      if (2 * t + 1 < nb) d[g + 1] = (uint16_t)scale_of(2 * t + 1);
    }
  }
}

// Q4_K super-blocks (144 bytes: d, dmin, 12 scale bytes, 128 code bytes) ->
// the planes of the Q4_K GEMM: the 16 leading bytes of super-block s to
// hdr + 16 s, its 128 code bytes, in the file's order, to w4 + 128 s (rows of
// w4 are K / 2 bytes, super-blocks of a row follow each other).  144 = 9 x 16,
// so with the blocks 16-byte aligned every 16-byte piece stays whole: thread
// p moves piece p % 9 of super-block p / 9 with one 16-byte load and store.
// Consecutive threads read consecutive pieces.
__global__ __launch_bounds__(256) void repack_q4_k_kernel(const uint8_t* __restrict__ blocks, uint8_t* __restrict__ w4,
                                                          uint8_t* __restrict__ hdr, int64_t npieces) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= npieces) return;
  const int64_t sb = p / 9;
  const int i = (int)(p - sb * 9);
  const v4i v = *reinterpret_cast<const v4i*>(blocks + 16 * p);
  uint8_t* dst = i == 0 ? hdr + 16 * sb : w4 + 128 * sb + 16 * (i - 1);
  *reinterpret_cast<v4i*>(dst) = v;
}

}  // namespace

int launch_repack_q4_k(const uint8_t* blocks, uint8_t* w4, uint8_t* hdr, int64_t N, int64_t K, hipStream_t st) {
  const int64_t npieces = N * (K / 256) * 9;
  repack_q4_k_kernel<<<(unsigned)((npieces + 255) / 256), 256, 0, st>>>(blocks, w4, hdr, npieces);
  return launch_status();
}

int launch_repack_q8_0(const uint8_t* blocks, int8_t* w, uint16_t* d, int64_t N, int64_t K, hipStream_t st) {
  const int64_t nblocks = N * (K / 32);
  const int64_t groups = (nblocks + kPerGroup - 1) / kPerGroup;
  repack_q8_0_kernel<<<(unsigned)groups, kPerGroup, 0, st>>>(blocks, w, d, nblocks);
  return launch_status();
}

}  // namespace prism
