// Control words of one fused-decode group and the protocol on them: the
// XCD placement mark, the two barrier forms, the final arrival that elects
// the merging workgroup, its status checks, and the reset that leaves the
// words zero for the next call.
//
// Words of a group (uint32, from the group's control base):
//   [1]            error word, device scope: bit 0 a wait timed out, bit 1
//                  the group's members sat on more than one XCD
//   [2], [3]       XCD-local form: arrival counter, and "a wait timed out"
//                  as seen in this L2
//   [16 + 16 w]    device-wide form: member w's flag (its own 64-byte line);
//                  XCD-local form: [16] is the placement mask
// Every wait is a bounded spin.  A member whose wait runs out sets the error
// word and s_fail; the caller then poisons its output.
#pragma once

#include <recsa_hw.hpp>

#include "recsa_common.hpp"

namespace recsa {

constexpr uint32_t kSpinLimit = 1u << 19;

struct FusedCtl {
  uint32_t* err;
  uint32_t* counter;    // counter[0] arrivals, counter[1] timed-out flag (same L2)
  uint32_t* flags;      // flags[16 w]; flags[0] also the placement mask
};

__device__ __forceinline__ FusedCtl fused_ctl(uint32_t* base) {
  return FusedCtl{base + 1, base + 2, base + 16};
}

// Value of *p read by an atomic executed in the L2 (a plain or relaxed
// workgroup-scope load may be served by this CU's L1).
__device__ __forceinline__ uint32_t l2_read(uint32_t* p) {
  uint32_t e = 0xFFFFFFFFu;
  __hip_atomic_compare_exchange_strong(p, &e, 0xFFFFFFFFu, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
  return e;
}

// Thread 0, XCD-local form: record this workgroup's XCD in the group's
// placement mask (device scope).  ctl_mark_xcd waits for the returned value;
// ctl_mark_xcd_post does not: it is performed before this workgroup's first
// arrival all the same, since the arrival first waits for every memory
// operation of the arriving wave (s_waitcnt 0), so other loads can be in
// flight with it (the fused decode issues its query loads right behind it).
__device__ __forceinline__ uint32_t ctl_mark_xcd_issue(const FusedCtl& c) {
  return __hip_atomic_fetch_or(c.flags, 1u << xcc_id(), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ctl_mark_xcd_post(const FusedCtl& c) {
  (void)ctl_mark_xcd_issue(c);
}
__device__ __forceinline__ void ctl_mark_xcd(const FusedCtl& c, uint32_t* s_fail) {
  const uint32_t prev = ctl_mark_xcd_issue(c);
  if (prev & 0x80000000u) *s_fail = 1u;     // never set: waits for the result
}

// XCD-local barrier.  Every wave drains its own memory operations, so after
// the workgroup barrier the workgroup's stores are in the XCD's L2; one
// thread adds this arrival to the group's counter (an L2 atomic), waits for
// `target` arrivals, and invalidates this CU's L1 so that later loads see
// what the other workgroups wrote.
__device__ __forceinline__ void group_barrier_xcd(uint32_t* counter, uint32_t target,
                                                  uint32_t* err, uint32_t* s_fail,
                                                  uint32_t spin_limit = kSpinLimit) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    uint32_t spins = 0;
    while (l2_read(counter) < target) {
      spin_pause();
      if (++spins > spin_limit) {
        atomicOr(err, 1u);                       // for the host (device scope)
        __hip_atomic_fetch_or(counter + 1, 1u, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);   // for the merge (this L2)
        *s_fail = 1u;
        break;
      }
    }
    l1_invalidate();
  }
  __syncthreads();
}

// Device-wide barrier.  After the workgroup barrier one thread releases the
// workgroup's stores to the device (one L2 write-back per workgroup), raises
// this workgroup's flag to `gen`, waits for every flag of the group with
// relaxed loads, and acquires once (one L2 invalidation per workgroup).
__device__ __forceinline__ void group_barrier(uint32_t* flags, int w, int W, uint32_t gen,
                                              uint32_t* err, uint32_t* s_fail,
                                              uint32_t spin_limit = kSpinLimit) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    // an atomic read-modify-write is performed where every XCD sees it (a
    // plain store could stay in this XCD's L2)
    __hip_atomic_exchange(flags + 16 * w, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every poll reads all W flags at once (one memory round trip)
    uint32_t spins = 0;
    while (true) {
      uint32_t lo = 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i < kFusedMaxW; ++i) {
        if (i < W)
          lo = min(lo, __hip_atomic_load(flags + 16 * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      }
      if (lo >= gen) break;
      spin_pause();
      if (++spins > spin_limit) {
        atomicOr(err, 1u);
        *s_fail = 1u;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Group status gathered by the merging workgroup.
struct FusedStatus {
  uint32_t mask = 0u;   // placement mask (XCD ids of the members)
  uint32_t late = 0u;   // a wait timed out in this L2
  uint32_t err = 0u;    // the sticky error word
};

// Thread 0, XCD-local form, after this workgroup's partial is written and
// drained: count its final arrival (the last of gen + 1 rounds of W).  The
// workgroup whose arrival completes the count merges: every partial is then
// in the L2.  It invalidates its L1 and reads the group's status words at
// once, so their latency overlaps the merge.
__device__ __forceinline__ bool xl_final_arrival(const FusedCtl& c, uint32_t gen, int W,
                                                 FusedStatus& st) {
  const uint32_t before =
      __hip_atomic_fetch_add(c.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const bool last = before + 1 == (gen + 1) * static_cast<uint32_t>(W);
  if (last) {
    l1_invalidate();
    st.mask = __hip_atomic_load(c.flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st.late = l2_read(c.counter + 1);
    st.err = __hip_atomic_load(c.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return last;
}

// Thread 0 of the merging workgroup (XCD-local form), after the merge:
// whether the result must be poisoned -- this member's or any member's
// timed-out wait (this L2's word, or device-wide the sticky error word), or
// members on more than one XCD (recorded in the error word).
__device__ __forceinline__ bool xl_result_bad(const FusedCtl& c, const FusedStatus& st,
                                              uint32_t s_fail) {
  const bool split = __popc(st.mask) != 1;
  if (split) atomicOr(c.err, 2u);
  return (s_fail | st.late | (split ? 1u : 0u) | st.err) != 0u;
}

// Thread 0 of the merging workgroup (XCD-local form): every workgroup has
// arrived for the last time, so none reads these words again.
__device__ __forceinline__ void xl_reset(const FusedCtl& c) {
  __hip_atomic_exchange(c.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __hip_atomic_exchange(c.counter + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __hip_atomic_exchange(c.flags, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 of member w > 0 (device-wide form), after its partial is written
// and drained: release it and raise the final flag gen + 1.
__device__ __forceinline__ void dw_final_flag(const FusedCtl& c, int w, uint32_t gen) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __hip_atomic_exchange(c.flags + 16 * w, gen + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-wide form, member 0 after its final wait and the merge: whether the
// result must be poisoned (its own timed-out wait or the sticky error word).
__device__ __forceinline__ bool dw_result_bad(const FusedCtl& c, uint32_t s_fail) {
  return s_fail || __hip_atomic_load(c.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Threads tid < W of member 0 (device-wide form): every other member has
// raised its final flag, so none reads them again.
__device__ __forceinline__ void dw_reset(const FusedCtl& c, int tid, int W) {
  if (tid < W) __hip_atomic_exchange(c.flags + 16 * tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace recsa
