// Direct global->LDS staging shared by the LDS-tiled MFMA kernels (gfx950).
#pragma once
#include "common.h"

namespace moe {
namespace {

#define MOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

template <int CH>
__device__ __forceinline__ int swz_ch(int row) {
  return row & (CH - 1);   // measured conflict-free on gfx950 for 16-row x 16-byte fragment reads
}
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ swz_ch<8>(row); }

// Direct global->LDS loads: lane l's bytes land at lds_base + size*l (M0 holds lds_base). They are
// issued from inline asm so that the compiler, which cannot tell which ring buffer a load
// targets, does not drain every outstanding load before each LDS read; the kernels wait for
// them explicitly (vmcnt) instead. The asm has no output registers. The compiler treats M0 as
// reserved and ignores the clobber, so this relies on the kernels that use these helpers having
// no M0 use of their own: tests/test_isa.py checks their gfx950 assembly for exactly that.
__device__ __forceinline__ void dma16(const void* g, uint8_t* lds_base) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(size_t)MOE_LDS(lds_base));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(base) : "memory", "m0");
}

// The same with the LDS byte address given directly (no generic-pointer conversion) and, for the
// saddr form, a uniform 64-bit base in SGPRs plus a per-lane 32-bit byte offset. NT: non-temporal.
template <bool NT>
__device__ __forceinline__ void dma16_at(const void* g, unsigned lds_addr) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(lds_addr) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr) : "memory", "m0");
}
template <bool NT>
__device__ __forceinline__ void dma16_sv(const void* base, unsigned voff, unsigned lds_addr) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(lds_addr)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr)
                 : "memory", "m0");
}

// the same, non-temporal (for data read once per launch, such as expert weights)
__device__ __forceinline__ void dma16_nt(const void* g, uint8_t* lds_base) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(size_t)MOE_LDS(lds_base));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(base) : "memory", "m0");
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's loads are outstanding, then a workgroup barrier without a
// memory fence (a fence would make the compiler drain every outstanding load, including the
// stages still in flight). Each wave's own wait plus the barrier make the stage's LDS data
// complete for all waves; every earlier LDS read has been consumed by an MFMA by then.
template <int N>
__device__ __forceinline__ void wait_dma_keep_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait until at most n (a runtime count in [LO, HI], uniform) of this wave's vector memory
// instructions are outstanding, then a barrier without a memory fence; a count outside the range
// waits for all of them.
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_n_barrier(int n) {
  if constexpr (LO > HI) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
    if (n == LO) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LO) : "memory");
    else wait_vm_n_barrier<LO + 1, HI>(n);
  }
}

// A barrier after this wave's LDS reads have returned (no wait on vector memory).
__device__ __forceinline__ void lds_reads_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void dma4(const void* g, float* lds_base) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(size_t)MOE_LDS(lds_base));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(base) : "memory", "m0");
}

}  // namespace
}  // namespace moe
