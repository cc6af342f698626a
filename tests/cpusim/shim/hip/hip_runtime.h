// Host stand-in for <hip/hip_runtime.h>, for building the selection device
// code (recsa_device.hpp) and the fused decode's control protocol
// (recsa_fused_ctl.hpp) on the CPU under sanitizers: each GPU lane is a
// host thread, a workgroup is NT such threads, and the wave-level operations
// (DPP moves, readlane) and barriers are emulated with std::barrier and a
// per-wave exchange array.  Only what the top-k path uses is modelled
// exactly; the other builtins exist so the header compiles.
#pragma once

#include <barrier>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <memory>
#include <vector>

#define __device__
#define __host__
#define __global__
#define __forceinline__ inline
#define __shared__
#define __launch_bounds__(...)

struct uint2 { uint32_t x, y; };
struct uint4 { uint32_t x, y, z, w; };
struct float2 { float x, y; };
struct float4 { float x, y, z, w; };
inline uint2 make_uint2(uint32_t x, uint32_t y) { return {x, y}; }
inline uint4 make_uint4(uint32_t x, uint32_t y, uint32_t z, uint32_t w) { return {x, y, z, w}; }
inline float2 make_float2(float x, float y) { return {x, y}; }
inline float4 make_float4(float x, float y, float z, float w) { return {x, y, z, w}; }

struct SimDim3 { unsigned x = 0, y = 0, z = 0; };

namespace cpusim {

// One simulated workgroup: NT lanes in waves of 64.
struct Block {
  int nt;
  std::barrier<> block_bar;
  std::vector<std::unique_ptr<std::barrier<>>> wave_bar;
  std::vector<int> xchg;                     // [wave][64]
  explicit Block(int n) : nt(n), block_bar(n), xchg(static_cast<size_t>(n)) {
    for (int w = 0; w < n / 64; ++w) wave_bar.emplace_back(std::make_unique<std::barrier<>>(64));
  }
};

inline thread_local Block* blk = nullptr;

}  // namespace cpusim

inline thread_local SimDim3 threadIdx;
inline thread_local SimDim3 blockIdx;
inline thread_local SimDim3 blockDim;
inline thread_local SimDim3 gridDim;

inline void __syncthreads() { cpusim::blk->block_bar.arrive_and_wait(); }

namespace cpusim {
inline int lane_() { return static_cast<int>(threadIdx.x & 63u); }
inline int wave_() { return static_cast<int>(threadIdx.x >> 6); }
// all 64 lanes of the wave publish a value, then read another lane's
inline int exchange(int v, int src_lane_or_neg, int fallback) {
  Block& b = *blk;
  const int w = wave_();
  b.xchg[w * 64 + lane_()] = v;
  b.wave_bar[w]->arrive_and_wait();
  const int r = src_lane_or_neg >= 0 ? b.xchg[w * 64 + src_lane_or_neg] : fallback;
  b.wave_bar[w]->arrive_and_wait();
  return r;
}
}  // namespace cpusim

// DPP move of gfx9: quad_perm, row_shl / row_shr / row_ror, row_bcast:15 and
// row_bcast:31; lanes whose source is invalid get `old` (bound_ctrl off),
// lanes in rows outside row_mask keep `old`.
inline int __builtin_amdgcn_update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask,
                                       bool bound_ctrl) {
  (void)bank_mask;
  const int lane = cpusim::lane_(), row = lane >> 4, li = lane & 15;
  int sl = -1;
  if (ctrl >= 0 && ctrl <= 0xFF) {
    sl = (lane & ~3) | ((ctrl >> (2 * (lane & 3))) & 3);
  } else if (ctrl >= 0x101 && ctrl <= 0x10F) {            // row_shl:n
    const int s = li + (ctrl - 0x100);
    sl = s < 16 ? row * 16 + s : -1;
  } else if (ctrl >= 0x111 && ctrl <= 0x11F) {            // row_shr:n
    const int s = li - (ctrl - 0x110);
    sl = s >= 0 ? row * 16 + s : -1;
  } else if (ctrl >= 0x121 && ctrl <= 0x12F) {            // row_ror:n
    sl = row * 16 + ((li - (ctrl - 0x120)) & 15);
  } else if (ctrl == 0x142) {                             // row_bcast:15
    sl = row > 0 ? (row - 1) * 16 + 15 : -1;
  } else if (ctrl == 0x143) {                             // row_bcast:31
    sl = row >= 2 ? 31 : -1;
  } else {
    std::abort();                                         // not modelled
  }
  const int v = cpusim::exchange(src, sl, bound_ctrl ? 0 : old);
  return ((row_mask >> row) & 1) ? v : old;
}

inline int __builtin_amdgcn_readlane(int v, int l) { return cpusim::exchange(v, l, 0); }
inline int __builtin_amdgcn_readfirstlane(int v) { return cpusim::exchange(v, 0, 0); }
inline void __builtin_amdgcn_wave_barrier() {
  cpusim::blk->wave_bar[cpusim::wave_()]->arrive_and_wait();
}
#define __builtin_amdgcn_fence(order, scope) __atomic_thread_fence(__ATOMIC_SEQ_CST)

// HIP's scoped atomics, as sequentially consistent host atomics (the CPU
// emulation checks the control protocol's logic, not the GPU memory model;
// the scope argument is ignored)
#ifndef __HIP_MEMORY_SCOPE_WORKGROUP
#define __HIP_MEMORY_SCOPE_WORKGROUP 3
#endif
#ifndef __HIP_MEMORY_SCOPE_AGENT
#define __HIP_MEMORY_SCOPE_AGENT 4
#endif
// (macros: host clang knows the __hip_atomic_* names as builtins)
#define __hip_atomic_fetch_add(p, v, order, scope) __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST)
#define __hip_atomic_fetch_or(p, v, order, scope) __atomic_fetch_or(p, v, __ATOMIC_SEQ_CST)
#define __hip_atomic_exchange(p, v, order, scope) __atomic_exchange_n(p, v, __ATOMIC_SEQ_CST)
#define __hip_atomic_load(p, order, scope) __atomic_load_n(p, __ATOMIC_SEQ_CST)
#define __hip_atomic_compare_exchange_strong(p, e, d, so, fo, scope) \
  __atomic_compare_exchange_n(p, e, d, false, __ATOMIC_SEQ_CST, __ATOMIC_SEQ_CST)
inline void __builtin_amdgcn_sched_barrier(int) {}
inline void __builtin_amdgcn_s_sleep(int) {}
inline void __builtin_amdgcn_s_waitcnt(int) {}

inline int atomicAdd(int* p, int v) { return __atomic_fetch_add(p, v, __ATOMIC_RELAXED); }
inline uint32_t atomicOr(uint32_t* p, uint32_t v) { return __atomic_fetch_or(p, v, __ATOMIC_SEQ_CST); }

inline float __expf(float x) { return std::exp(x); }
inline float __builtin_amdgcn_exp2f(float x) { return std::exp2(x); }
inline int __clz(int x) { return x == 0 ? 32 : __builtin_clz(static_cast<unsigned>(x)); }
inline int __popc(unsigned x) { return __builtin_popcount(x); }
inline float __uint_as_float(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
inline uint32_t __float_as_uint(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
inline float __int_as_float(int u) { float f; std::memcpy(&f, &u, 4); return f; }
inline int __float_as_int(float f) { int u; std::memcpy(&u, &f, 4); return u; }
inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }
inline uint32_t min(uint32_t a, uint32_t b) { return a < b ? a : b; }
inline uint32_t max(uint32_t a, uint32_t b) { return a > b ? a : b; }
inline int64_t min(int64_t a, int64_t b) { return a < b ? a : b; }
inline int64_t max(int64_t a, int64_t b) { return a > b ? a : b; }

// present so the header compiles; the top-k path never calls them
typedef __bf16 cpusim_bf16x2 __attribute__((ext_vector_type(2)));
inline float __builtin_amdgcn_fdot2_f32_bf16(cpusim_bf16x2, cpusim_bf16x2, float acc, bool) {
  std::abort();
  return acc;
}
typedef __bf16 cpusim_bf16x8 __attribute__((ext_vector_type(8)));
typedef float cpusim_f32x4 __attribute__((ext_vector_type(4)));
inline cpusim_f32x4 __builtin_amdgcn_mfma_f32_16x16x32_bf16(cpusim_bf16x8, cpusim_bf16x8,
                                                            cpusim_f32x4 c, int, int, int) {
  std::abort();
  return c;
}
typedef uint32_t cpusim_u32x2 __attribute__((ext_vector_type(2)));
inline cpusim_u32x2 __builtin_amdgcn_permlane16_swap(uint32_t a, uint32_t, bool, bool) {
  std::abort();
  return cpusim_u32x2{a, a};
}
inline cpusim_u32x2 __builtin_amdgcn_permlane32_swap(uint32_t a, uint32_t, bool, bool) {
  std::abort();
  return cpusim_u32x2{a, a};
}
inline float __shfl_xor(float v, int, int = 64) { std::abort(); return v; }
inline float __shfl(float v, int, int = 64) { std::abort(); return v; }
inline uint32_t __shfl(uint32_t v, int, int = 64) { std::abort(); return v; }
