// Building blocks of the pipelined MFMA kernels (gfx950): bf16 fragments,
// direct global->LDS loads with exact vector-memory waits, and the LDS row
// swizzle of 64-deep k-tiles.
#pragma once

#include "omni_internal.h"

namespace omni {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 counts loads and stores together, in issue order).
template <int N>
__device__ __forceinline__ void wait_vm_imm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most i * N of this wave's vector loads are outstanding
// (i = 0 .. MAXI, the k-tiles allowed to stay in flight; N loads per k-tile).
template <int N, int MAXI>
__device__ __forceinline__ void wait_vm_tiles(int i) {
  if constexpr (MAXI >= 3) {
    if (i >= 3) return wait_vm_imm<3 * N>();
  }
  if constexpr (MAXI >= 2) {
    if (i >= 2) return wait_vm_imm<2 * N>();
  }
  if constexpr (MAXI >= 1) {
    if (i >= 1) return wait_vm_imm<N>();
  }
  wait_vm_imm<0>();
}

// Workgroup barrier without the fence of __syncthreads (which would also
// wait for every direct-to-LDS load still in flight).
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte chunk c of LDS row r sits in slot c ^ chunk_swz(r): the 16 rows
// read by one ds_read_b128 of an MFMA operand fall in distinct bank groups.
template <int BK>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (BK == 64) return (r >> 1) & 7;  // 8 chunks per 128-byte row
  else return (r >> 2) & 3;                     // 4 chunks per 64-byte row
}

}  // namespace omni
