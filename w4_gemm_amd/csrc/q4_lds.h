// q4_lds.h -- the pieces the LDS-staged kernels share on gfx950: direct
// global->LDS copies (global_load_lds_dword[x4]: each lane's bytes land at
// the wave-uniform LDS base + lane * size, with no register round trip),
// explicit s_waitcnt counts for them, and a barrier that orders LDS accesses
// without draining the copies still in flight.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// each lane copies 16 (4) bytes from src to lds_base + 16 (4) * lane;
// lds_base must be wave-uniform
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)lds_base, 4, 0, 0);
}

// A wave-uniform pointer held in scalar registers (readfirstlane), so that
// adding the lane offset at each copy cannot be hoisted into per-lane
// 64-bit registers for the whole loop.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// s_waitcnt vmcnt(N) with no wait on the other counters (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  Loads, including
// the LDS copies, complete in issue order, so N = the number of loads
// issued after the ones to wait for.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));
}

// Workgroup barrier that does not wait for outstanding copies (each wave
// has waited for its own, by count, before it).  The empty asm statements
// and scheduling barriers keep the compiler from moving memory accesses or
// instructions across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// The same barrier without the scheduling barriers: only memory accesses
// stay on their side, arithmetic may move across (the W4A4 kernel measured
// 2-4% faster with this one).
__device__ __forceinline__ void stage_barrier_loose() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace q4
