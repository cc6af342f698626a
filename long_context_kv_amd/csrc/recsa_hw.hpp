// The three hardware operations the fused decode's control code issues
// directly: this CU's L1 invalidation, the id of the XCD the workgroup runs
// on, and a short sleep between polls.  (Kept in a header of their own: the
// CPU emulation of the control protocol supplies host versions of exactly
// these.)
#pragma once

#include <hip/hip_runtime.h>

namespace recsa {

// Invalidate this CU's L1 so that later loads see what other workgroups
// left in the shared L2.
__device__ __forceinline__ void l1_invalidate() {
  __asm__ __volatile__("buffer_inv sc0" ::: "memory");
}

// hwreg XCC_ID: the XCD this workgroup was placed on.
__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg(20 | (15 << 11)) & 0xF;
}

__device__ __forceinline__ void spin_pause() { __builtin_amdgcn_s_sleep(1); }

}  // namespace recsa
