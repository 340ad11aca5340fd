// Direct global->LDS loads and explicit pipeline waits for gfx950 kernels.
//
// global_load_lds_dword(x4) writes each lane's data to LDS at M0 + size*lane,
// so one wave fills a contiguous block from 64 arbitrary global addresses.
// The loads are issued from inline assembly: the compiler then leaves their
// completion to the kernel, which waits with an explicit vmcnt before the
// barrier that publishes a stage (the compiler would otherwise wait for every
// outstanding LDS DMA before any LDS read, serialising the pipeline).  The
// helpers write M0, a register the compiler reserves and does not let inline
// assembly clobber; the kernels that use them never index register arrays
// dynamically, and a CPU test (test_codegen.py) checks the compiled code: no
// instruction outside these helpers reads or writes M0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace nms {

__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}
// dma16 by the lanes below `lanes` only (1 <= lanes <= 64).  The other lanes are masked off in
// EXEC inside the same assembly block, which restores EXEC before it ends: the wave issues exactly
// one load whatever the lane count, with no branch around it, so every wave's count of
// outstanding vector-memory operations is the same fixed number.
__device__ __forceinline__ void dma16_lanes(const void* g, uint32_t lds, uint64_t lane_mask) {
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\ts_mov_b64 exec, %2\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lane_mask), "s"(lds)
      : "memory");
}
// The same with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit byte offset: one VGPR
// per source instead of two.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Loads into registers from inline assembly: the compiler does not count them, so a kernel waits
// with wait_vmcnt_regs, whose in/out register operands keep every reader of the destination
// after the wait.  (tests/test_codegen.py checks the compiled kernels: nothing touches a
// destination register before a wait has retired its load.)
__device__ __forceinline__ u32x4 load16_async(const void* g) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(g));
  return r;
}
template <int N>
__device__ __forceinline__ void wait_vmcnt_regs(u32x4 (&rb)[8]) {
  asm volatile("s_waitcnt vmcnt(%8)"
               : "+v"(rb[0]), "+v"(rb[1]), "+v"(rb[2]), "+v"(rb[3]), "+v"(rb[4]), "+v"(rb[5]), "+v"(rb[6]),
                 "+v"(rb[7])
               : "n"(N)
               : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt_regs(u32x4 (&r0)[8], u32x4 (&r1)[8]) {
  asm volatile("s_waitcnt vmcnt(%16)"
               : "+v"(r0[0]), "+v"(r0[1]), "+v"(r0[2]), "+v"(r0[3]), "+v"(r0[4]), "+v"(r0[5]), "+v"(r0[6]),
                 "+v"(r0[7]), "+v"(r1[0]), "+v"(r1[1]), "+v"(r1[2]), "+v"(r1[3]), "+v"(r1[4]), "+v"(r1[5]),
                 "+v"(r1[6]), "+v"(r1[7])
               : "n"(N)
               : "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
// Barrier that first waits for this wave's LDS reads and writes (and scalar loads): after it,
// every wave's LDS writes issued before it are visible and its LDS reads have completed.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace nms
