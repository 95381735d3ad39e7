// Low-level helpers shared by the gfx950 kernels: direct-to-LDS DMA, vmcnt
// waits and a workgroup barrier without a memory fence. Device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

namespace blkattn {

// s_waitcnt vmcnt(n) leaving the other counters free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would drain every outstanding DMA (vmcnt(0)) at each tile. LDS data is
// ordered explicitly instead: DMA completion by s_waitcnt vmcnt before the
// barrier, and every LDS read of a tile is consumed by an MFMA before the
// barrier that lets its slot be refilled. The scheduling barriers keep the
// compiler from moving any instruction across it.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// One direct-to-LDS DMA: 64 lanes x 16 bytes from per-lane global addresses
// into 1 KB of LDS at lds_addr (wave-uniform, through M0). A scalar write of
// M0 needs one wait state before an LDS-DMA load reads it (the s_nop 0, which
// the compiler cannot insert inside one asm statement). Written as inline
// asm so that the compiler does not see an LDS write in flight and drain the
// whole DMA ring (vmcnt(0)) before every LDS read; completion is ordered
// explicitly by vmcnt waits before the tile barriers. The instruction has no
// register results. NT marks the load non-temporal (streamed once: the caches
// need not keep it), which lets a long single-pass stream run faster.
template <bool NT = false>
__device__ __forceinline__ void dma_1k(const void* gptr, uint32_t lds_addr) {
  if constexpr (NT) {
    __asm__ __volatile__(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr)
        : "memory", "m0");
  } else {
    __asm__ __volatile__(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr)
        : "memory", "m0");
  }
}

// The same DMA from a wave-uniform base in scalar registers plus a per-lane
// unsigned 32-bit byte offset.
template <bool NT = false>
__device__ __forceinline__ void dma_1k_s(const char* sbase, uint32_t voff, uint32_t lds_addr) {
  if constexpr (NT) {
    __asm__ __volatile__(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(sbase)
        : "memory", "m0");
  } else {
    __asm__ __volatile__(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(sbase)
        : "memory", "m0");
  }
}

// Four DMAs of 1 KB from a wave-uniform base in scalar registers: DMA i reads
// 16 bytes per lane at sbase + voff_i + 1024*i and writes them to LDS at
// lds_addr + 1024*i + 16*lane. The instruction offset moves the global and
// the LDS address alike, so the four share one M0 write and one base.
template <bool NT = false>
__device__ __forceinline__ void dma_4k_s(const char* sbase, uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                         uint32_t lds_addr) {
  if constexpr (NT) {
    __asm__ __volatile__(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %5 nt\n\t"
        "global_load_lds_dwordx4 %2, %5 offset:1024 nt\n\t"
        "global_load_lds_dwordx4 %3, %5 offset:2048 nt\n\t"
        "global_load_lds_dwordx4 %4, %5 offset:3072 nt"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(sbase)
        : "memory", "m0");
  } else {
    __asm__ __volatile__(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %5\n\t"
        "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
        "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
        "global_load_lds_dwordx4 %4, %5 offset:3072"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(sbase)
        : "memory", "m0");
  }
}

// A wave-uniform pointer moved to scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* q) {
  const uint64_t v = (uint64_t)(uintptr_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// A value hidden from the optimiser: what is computed from it is recomputed
// where it is used instead of being hoisted out of the tile loop and kept in
// registers (or spilled) through it.
__device__ __forceinline__ int opaque(int x) {
  __asm__ __volatile__("" : "+v"(x));
  return x;
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)LDS_PTR(const char, ptr);
}

// Wait until at most n (wave-uniform) of this wave's loads are in flight,
// n rounded down to the nearest of the counts N, Rest... (descending, ending
// with 0): waiting for fewer in flight than allowed is always safe.
template <int N, int... Rest>
__device__ __forceinline__ void wait_at_most(int n) {
  if constexpr (sizeof...(Rest) == 0) {
    static_assert(N == 0, "the last count is 0");
    wait_vm<0>();
  } else {
    if (n >= N) wait_vm<N>();
    else wait_at_most<Rest...>(n);
  }
}

}  // namespace blkattn
