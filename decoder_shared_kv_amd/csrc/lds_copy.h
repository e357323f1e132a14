// Device helpers shared by the kernels that stream tiles HBM -> LDS with the
// load unit (global_load_lds_dwordx4) and wait for them by count.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define YOCO_LDS __attribute__((address_space(3)))

namespace yoco {

// s_waitcnt with vmcnt = n and lgkmcnt = 0 (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 left at its maximum, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without the memory fence of __syncthreads (which would also
// wait for the tiles still in flight); the empty asm keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// HBM -> LDS copies by the load unit: 16 bytes per lane (lane l's land at
// dst + 16 l; dst is wave-uniform), or 4 (dma4). Written as asm so that the compiler does
// not count them among its own LDS events (which would make it wait for every
// LDS read to finish before the next MFMA); their completion is awaited
// explicitly with s_waitcnt vmcnt before the workgroup barrier of their tile.
// The s_nop covers the wait states a load-to-LDS needs after an M0 write (and
// after a VALU write of an SGPR operand), which the compiler does not insert
// inside asm. Kernels that use these must not use M0 otherwise.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved; the kernels using this leave it alone
// per-lane 64-bit source address
__device__ __forceinline__ void dma16(const void* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(dst), "v"(src) : "memory", "m0");
}
// wave-uniform 64-bit base + per-lane 32-bit byte offset: no per-lane address arithmetic
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(dst), "v"(off), "s"(base)
               : "memory", "m0");
}
// ... the same with the nontemporal hint, for data read once and not again soon
// (streamed through the caches without displacing what is reused)
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(dst), "v"(src)
               : "memory", "m0");
}
// 4 bytes per lane (lane l's dword lands at dst + 4 l), per-lane 64-bit source address
__device__ __forceinline__ void dma4(const void* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dword %1, off" ::"s"(dst), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace yoco
