// LDS and direct-to-LDS load helpers of the MFMA kernels (gfx950, wave64).
#pragma once

#include "common.h"

namespace moe {

typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// Transposing LDS read: within each 16-lane group, lane i receives element
// i%4 of the 8-byte chunks read by lanes 4r + i/4, r = 0..3.
__device__ __forceinline__ short4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p));
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maximum, i.e. not waited for).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ... and additionally until every LDS read of this wave has returned.
template <int n>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
}

// A wave-uniform pointer, moved to scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// One wave-wide direct-to-LDS load: lane l copies the 16 bytes at
// base + voff (base wave-uniform, voff the lane's byte offset) to
// lds + 16*l; M0 holds the wave's LDS destination. Written as inline
// assembly: the compiler's own LDS-DMA tracking cannot tell the ring buffers
// apart for every LDS read and would drain all loads in flight before it,
// while the kernel waits for exactly the stage it needs (vmcnt). An LDS
// byte's generic address is the LDS aperture's base in the upper 32 bits and
// the LDS address in the lower 32, so the lower half is M0's value: a
// generic-to-LDS cast would give the same for the (never null) ring
// buffers, plus a null test and a 64-bit readfirstlane per instruction.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, char* lds) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  asm volatile("global_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(uniform(base)), "{m0}"(__builtin_amdgcn_readfirstlane(m0))
               : "memory");
}

}  // namespace moe
