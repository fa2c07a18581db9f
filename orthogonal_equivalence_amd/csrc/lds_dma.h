// Device helpers for kernels that copy global memory straight into LDS
// (global_load_lds_dwordx4, gfx950) and read it back with plain or
// transposing LDS loads.
#pragma once

#include "common.h"

namespace poetx {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) void lds_void;

// One global_load_lds_dwordx4: every lane copies 16 bytes from gptr into LDS
// at lds_base + 16 * lane. Issued through inline assembly so that the only
// waits on it are the explicit s_waitcnt of the caller's pipeline.
__device__ __forceinline__ void dma16(const void* gptr, const bf16_t* lds_base) {
  // lds_base is the same for the whole wave; make that explicit for the SGPR
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)lds_base)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(gptr)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) leaving the other counters unconstrained (gfx9 encoding).
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding global load). The empty asm keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ds_read_b64_tr_b16 of a row-major [k][n] bf16 tile: within each group of
// 16 lanes, when lane j addresses the 8 bytes at (k0 + j / 4, n0 + 4 (j % 4)),
// lane i receives the column entries (k0 + q, n0 + i), q = 0..3.
__device__ __forceinline__ short4_t ds_read_tr4(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
}

}  // namespace poetx
