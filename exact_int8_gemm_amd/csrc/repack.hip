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

// Q4_K super-blocks (public GGUF layout, 144 bytes per 256 weights): binary16
// d and dmin, 12 bytes of 6-bit sub-block scales sc_j and mins m_j, 128 bytes
// of 4-bit codes (byte 32 g + l: weight 64 g + l in the low nibble, weight
// 64 g + 32 + l in the high one).  Output planes: the codes as int8 [N][K]
// (0..15), D = d * sc_j and Mn = dmin * m_j as fp32 [N][K/32]; both products
// are exact in fp32 (11 + 6 significant bits).  One workgroup moves 64
// super-blocks (9216 bytes, a whole number of 16-byte pieces, each
// super-block 16-byte aligned) through LDS.
constexpr int kQ4kBytes = 144;
constexpr int kQ4kPerGroup = 64;

__global__ __launch_bounds__(256) void repack_q4_k_kernel(const uint8_t* __restrict__ blocks, int8_t* __restrict__ w,
                                                          float* __restrict__ D, float* __restrict__ Mn,
                                                          int64_t nsuper) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[kQ4kPerGroup * kQ4kBytes];
  const int64_t s0 = (int64_t)blockIdx.x * kQ4kPerGroup;
  const int ns = nsuper - s0 < kQ4kPerGroup ? (int)(nsuper - s0) : kQ4kPerGroup;
  const uint32_t nbytes = (uint32_t)ns * kQ4kBytes;  // a multiple of 16
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blocks + s0 * kQ4kBytes), (short)0, (int)nbytes,
                                        0x00020000);
  for (uint32_t i = threadIdx.x; i < nbytes / 16; i += 256)
    *reinterpret_cast<v4i*>(buf + 16 * i) = __builtin_amdgcn_raw_buffer_load_b128(r, i * 16, 0, 0);
  __syncthreads();

  // Codes: piece h covers codes 16 h' .. 16 h' + 15 of super-block h / 16 (h' = h % 16),
  // all within one half of one 64-code group, so one 16-byte read of qs gives them.
  for (int h = threadIdx.x; h < ns * 16; h += 256) {
    const int sb = h >> 4, k0 = (h & 15) * 16, g = k0 >> 6, l = k0 & 63;
    const v4i v = *reinterpret_cast<const v4i*>(buf + sb * kQ4kBytes + 16 + 32 * g + (l & 31));
    v4i o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (int)(l < 32 ? ((uint32_t)v[e] & 0x0f0f0f0fu) : (((uint32_t)v[e] >> 4) & 0x0f0f0f0fu));
    *reinterpret_cast<v4i*>(w + (s0 + sb) * 256 + k0) = o;
  }
  // Scales: thread t handles sub-blocks 2 (t % 4) and 2 (t % 4) + 1 of super-block t / 4.
  const int t = threadIdx.x, sb = t >> 2;
  if (sb < ns) {
    const uint8_t* b = buf + sb * kQ4kBytes;
    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(b[0] | (b[1] << 8)));
    const float dmin = (float)__builtin_bit_cast(_Float16, (uint16_t)(b[2] | (b[3] << 8)));
    const uint8_t* sc = b + 4;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = 2 * (t & 3) + e;
      int c, m;
      if (j < 4) {
        c = sc[j] & 63;
        m = sc[j + 4] & 63;
      } else {
        c = (sc[j + 4] & 15) | ((sc[j - 4] >> 6) << 4);
        m = (sc[j + 4] >> 4) | ((sc[j] >> 6) << 4);
      }
      D[(s0 + sb) * 8 + j] = d * (float)c;
      Mn[(s0 + sb) * 8 + j] = dmin * (float)m;
    }
  }
}

}  // namespace

int launch_repack_q4_k(const uint8_t* blocks, int8_t* w, float* D, float* Mn, int64_t N, int64_t K, hipStream_t st) {
  const int64_t nsuper = N * (K / 256);
  const int64_t groups = (nsuper + kQ4kPerGroup - 1) / kQ4kPerGroup;
  repack_q4_k_kernel<<<(unsigned)groups, 256, 0, st>>>(blocks, w, D, Mn, nsuper);
  return launch_status();
}

int launch_repack_q8_0(const uint8_t* blocks, int8_t* w, uint16_t* d, int64_t N, int64_t K, hipStream_t st) {
  const int64_t nblocks = N * (K / 32);
  const int64_t groups = (nblocks + kPerGroup - 1) / kPerGroup;
  repack_q8_0_kernel<<<(unsigned)groups, kPerGroup, 0, st>>>(blocks, w, d, nblocks);
  return launch_status();
}

}  // namespace prism
