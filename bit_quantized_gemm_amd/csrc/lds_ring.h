// LDS stage rings for the gfx950 GEMM kernels (gemm.hip, gemm_w4a8.hip): copies from global
// memory straight into LDS, the waits and barriers of a ring of stage buffers, and the
// compile-time unrolling that keeps every buffer index a constant.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace atom {

// s_waitcnt immediate (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8): wait until at
// most n vector-memory operations of this wave are outstanding and all its LDS operations
// have completed.  n = 63 leaves vector memory alone.
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Workgroup barrier that does not wait for this wave's outstanding vector-memory operations
// (__syncthreads would drain every copy in flight).  The empty asm statements keep the
// compiler from moving memory operations across it; callers wait for what must be complete.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One LDS-DMA instruction: lane i loads 16 bytes at voff + soff of the buffer and writes them
// to lds + 16 i (lds is wave-uniform).  Not a template: the LDS address-space cast exists
// only for the device.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Compile-time ring position of a stage buffer in a ring of NB buffers.
template <int P, int NB>
struct Ring {
  static constexpr int kCur = P, kNext = (P + 1) % NB, kAfterNext = (P + 2) % NB;
};

// f(Ring<P, NB>, s + P) for P = 0 .. NB-1: one turn of the ring, every buffer index a constant.
template <int P, int NB, class F>
__device__ __forceinline__ void ring_turn(F& f, int s) {
  if constexpr (P < NB) {
    f(Ring<P, NB>{}, s + P);
    ring_turn<P + 1, NB>(f, s);
  }
}
// The same for the groups s .. gb-1 left after the whole turns (fewer than NB).
template <int P, int NB, class F>
__device__ __forceinline__ void ring_tail(F& f, int s, int gb) {
  if constexpr (P < NB - 1) {
    if (s + P < gb) {
      f(Ring<P, NB>{}, s + P);
      ring_tail<P + 1, NB>(f, s, gb);
    }
  }
}

}  // namespace atom
