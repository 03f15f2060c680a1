// ring.h -- LDS DMA ring helpers shared by the MFMA kernels (gfx950).
//
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory to
// consecutive LDS addresses (lane i at base + 16 i; the base is wave-uniform).
// A ring stage is filled by such copies; each wave waits for its own copies
// with s_waitcnt vmcnt, then a bare workgroup barrier publishes the stage and
// guarantees that the slot refilled next has been read by every wave.
#pragma once

#include <hip/hip_runtime.h>

namespace mhc {

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void dma16(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds_base, 16, 0, 0);
}
// The same with the non-temporal cache policy, for a stream read once.
__device__ __forceinline__ void dma16_nt(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds_base, 16, 0, 2);
}

// s_waitcnt with vmcnt <= n (expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// vmcnt <= n for a wave-uniform n of at most 16; other values wait for all.
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n) {
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// LDS reads done, then a workgroup barrier.  The memory clobber keeps the
// compiler from moving LDS accesses across it; unlike __syncthreads it does
// not wait for copies still in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Orders this wave's LDS writes before its following LDS reads (the region
// is private to the wave, so no workgroup barrier is needed).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace mhc
