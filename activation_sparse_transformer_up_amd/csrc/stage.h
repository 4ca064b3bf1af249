// Synchronisation helpers of the LDS-staged MFMA loops (the up GEMM and the N:M down
// projection): vector-memory waits, workgroup barriers, and the ordering of one wave's LDS
// phases.
#pragma once
#include "common.h"

namespace tw {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N> TW_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

TW_DEV void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier after this wave's LDS reads have completed (lgkmcnt(0)), so that no read of a
// stage can still be pending when another wave's loads overwrite it.
TW_DEV void block_barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Ordering of one wave's own LDS accesses across the phases of an epilogue (pad, scatter,
// copy-out). A wave's LDS instructions execute in issue order, so only the compiler must be
// kept from moving accesses across the phase boundary; a memory fence would also wait for
// the wave's outstanding global stores (vmcnt(0)) and serialize the copy-out of every block.
TW_DEV void wave_lds_order() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace tw
