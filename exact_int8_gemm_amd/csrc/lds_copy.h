// Direct-to-LDS copies and the buffer resources they read through, shared
// by the tiled kernels and the small-M block kernels.
#pragma once

#include "prism_internal.h"

namespace prism {
namespace tiled {

// Byte offset that a buffer access treats as out of range: loads return 0.
constexpr uint32_t kOutOfRange = 0x80000000u;

namespace dma {

// Raw buffer resource as four dwords (raw, stride 0): base address, bounds
// `bytes` (clamped below kOutOfRange), data format word of gfx9.
__device__ inline v4i rsrc_words(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int64_t n = bytes < (int64_t)kOutOfRange - 1 ? bytes : (int64_t)kOutOfRange - 1;
  return v4i{(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xFFFFu), (int)n, 0x00020000};
}

// One wave-wide 16-byte-per-lane copy from a buffer into LDS at lds_addr +
// 16 * lane.  Written as inline assembly so that the compiler does not add
// its own (conservative) waits for it: every copy is awaited explicitly with
// wait_vmcnt before its data is read, and all are drained before the kernel
// leaves the main loop.  M0 (the LDS address of the copy) is written inside
// the same statement, right before the copy, and is declared as an output of
// the statement, so the compiler knows M0 is overwritten.  The compiler does
// not see that the statement holds an LDS DMA, so it must not be the one to
// place the M0 write: with M0 given as an input operand it put the next
// copy's M0 write directly behind a copy in flight, and the GPU faulted.
__device__ inline void copy_to_lds(const v4i rsrc, uint32_t lds_addr, uint32_t voff) {
  // lds_addr and rsrc are wave-uniform; readfirstlane puts them in SGPRs.
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  const v4i r = v4i{__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                    __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  uint32_t m0_out;
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds" : "={m0}"(m0_out) : "s"(m0v), "v"(voff), "s"(r) : "memory");
  (void)m0_out;
}

// The same for 2-byte elements: lane i's value lands zero-extended in the
// dword at lds_addr + 4 * lane.
__device__ inline void copy2_to_lds(const v4i rsrc, uint32_t lds_addr, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  const v4i r = v4i{__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                    __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  uint32_t m0_out;
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_ushort %2, %3, 0 offen lds" : "={m0}"(m0_out) : "s"(m0v), "v"(voff), "s"(r) : "memory");
  (void)m0_out;
}

// The same for 4-byte elements: lane i's dword lands at lds_addr + 4 * lane.
__device__ inline void copy4_to_lds(const v4i rsrc, uint32_t lds_addr, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  const v4i r = v4i{__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                    __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  uint32_t m0_out;
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dword %2, %3, 0 offen lds" : "={m0}"(m0_out) : "s"(m0v), "v"(voff), "s"(r) : "memory");
  (void)m0_out;
}

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ inline uint32_t lds_addr(const int8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int8_t*)p;
}

}  // namespace dma
}  // namespace tiled
}  // namespace prism
