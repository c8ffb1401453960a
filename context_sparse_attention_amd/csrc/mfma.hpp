// bf16 32x32x16 MFMAs with the register file of each operand chosen explicitly.
//
// In the attention key loops the compiler left to itself places score and
// output accumulators in whichever file it likes and then copies them between
// AGPRs and VGPRs on every tile.  These forms pin the classes: scores (and
// their A/B operands) in VGPRs, output accumulators in AGPRs.
//
// The compiler cannot see the MFMA's latency through inline assembly, so the
// forms carry the wait states themselves: each MFMA starts with the wait a
// preceding VALU write of its operands needs (1 on gfx950; 2 issued), and the
// fences separate the last MFMA writing a register from VALU accesses of it
// (the compiler inserts 12 for a 32x32x16 result; the fences issue 16 and 24).
// Back-to-back accumulation into the same registers needs no wait.
#pragma once

#include <hip/hip_runtime.h>

namespace csa {

// acc = A * B (scores in VGPRs)
template <typename V16, typename B8>
__device__ __forceinline__ void mfma_v0(V16& acc, const B8& a, const B8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
// acc += A * B (scores in VGPRs)
template <typename V16, typename B8>
__device__ __forceinline__ void mfma_v(V16& acc, const B8& a, const B8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// acc += A * B (output accumulators in AGPRs)
template <typename V16, typename B8>
__device__ __forceinline__ void mfma_a(V16& acc, const B8& a, const B8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states after the last MFMA writing these VGPR accumulators.
template <typename V16, int N>
__device__ __forceinline__ void fence_v(V16 (&acc)[N]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc[0]));
#pragma unroll
  for (int i = 1; i < N; ++i) asm volatile("" : "+v"(acc[i]));
}
// Wait states after the last MFMA writing these AGPR accumulators.
template <typename V16, int N>
__device__ __forceinline__ void fence_a(V16 (&acc)[N]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0]));
#pragma unroll
  for (int i = 1; i < N; ++i) asm volatile("" : "+a"(acc[i]));
}
// Hands the compiler a copy of v that lives in AGPRs (initial accumulator values).
template <typename V16>
__device__ __forceinline__ void to_agpr(V16& dst, const V16& v) {
  asm volatile("; to AGPRs" : "=a"(dst) : "0"(v));
}

}  // namespace csa
