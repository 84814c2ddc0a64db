// Direct global -> LDS loads (gfx950 global_load_lds_dwordx4) and the waits
// that order them, shared by the projection GEMM and the attention kernel.
#pragma once

#include <hip/hip_runtime.h>

namespace mha {

// One wave instruction moving 16 bytes per lane from global memory straight
// into LDS: lane i reads base + off (off per lane) and its bytes land at
// LDS address m0 + 16 i (m0 wave-uniform).  Written as inline assembly so
// the compiler does not see an LDS write in flight (it would otherwise wait
// for every such load before any LDS read); the kernels order these loads
// with explicit counter waits and barriers.  M0 is written only here (no
// other code of the kernels uses it); the s_nop covers the M0-write ->
// LDS-DMA hazard.
__device__ __forceinline__ void lds_dma16(const void* base, unsigned off, unsigned m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are
// outstanding and all its LDS operations have completed.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" : : : "memory"); }

}  // namespace mha
