// Direct global -> LDS gathers (global_load_lds_dwordx4) issued as assembly.
//
// One instruction fills 1 KiB of LDS from m0 on, lane l writing bytes
// [16 l, 16 l + 16), read from base + off (SGPR base, per-lane 32-bit offset).
// Issued as assembly so that the compiler does not see an LDS store: it would
// otherwise wait for the gather before every later LDS read, including reads
// of the tile being computed while the next one is gathered.  Users read a
// gathered tile only after wait_gathers() and a barrier.  The kernels that use
// these helpers make no other use of m0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

__device__ __forceinline__ void gather16(uint32_t off, const char* base, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds_dst)
               : "memory", "m0");
}

// The same gather with a full 64-bit address per lane (rows of different
// tokens within one 1 KiB chunk, where no common base exists).
__device__ __forceinline__ void gather16_addr(const void* src, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_dst)
               : "memory", "m0");
}

// s_waitcnt vmcnt(0) (gfx9 encoding, the other counters left alone)
__device__ __forceinline__ void wait_gathers() {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const char* lds_bytes;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_bytes)p));
}

}  // namespace csa
