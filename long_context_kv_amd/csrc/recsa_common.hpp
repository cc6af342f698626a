// Device helpers shared by the RecSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "recsa.h"

namespace recsa {

constexpr int kWave = 64;
constexpr int kBlock = 256;        // 4 waves per workgroup
constexpr int kC = 16;             // branching factor (picx.dev Tree Construction)
constexpr int kMaxK = 512;         // largest selection depth k
// A partial softmax state of one query head: max, sum, two unused floats,
// then the D weighted values (16-byte aligned for vector loads).
constexpr int kPartHead = 4;
constexpr int kMaxCK = 8192;       // longest candidate list, C*k
constexpr int kMaxG = 8;           // query heads per KV head
constexpr int kFusedMaxW = 32;     // workgroups per (sequence, KV head), fused decode
constexpr int kChunk = 256;        // list positions per attention/score chunk

// Rows allocated at a level: floor(L_cap / 16^level).
__host__ __device__ __forceinline__ int64_t level_rows_dev(int64_t L_cap, int level) {
  return L_cap >> (4 * level);
}

// ---------------------------------------------------------------- storage
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float32 -> bfloat16 bits (gfx950 converts in one
// instruction, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two float32 values rounded to bf16 (to nearest, ties to even, as
// f32_to_bf16_bits) and packed, lo in bits 0-15: one v_cvt_pk_bf16_f32.
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_convertvector((f32x2_cvt_t){lo, hi}, bf16x2_cvt_t));
}

template <int DT>
struct Stor;

template <>
struct Stor<RECSA_F32> {
  using T = float;
  static __device__ __forceinline__ float load(const T* p) { return *p; }
  static __device__ __forceinline__ void store(T* p, float v) { *p = v; }
  static __device__ __forceinline__ float round(float v) { return v; }
};

template <>
struct Stor<RECSA_BF16> {
  using T = uint16_t;
  static __device__ __forceinline__ float load(const T* p) { return bf16_bits_to_f32(*p); }
  static __device__ __forceinline__ void store(T* p, float v) { *p = f32_to_bf16_bits(v); }
  static __device__ __forceinline__ float round(float v) {
    return bf16_bits_to_f32(f32_to_bf16_bits(v));
  }
};

// Load n consecutive storage elements (n = 2, 4 or 8) as floats.
template <int DT, int N>
__device__ __forceinline__ void load_vec(const typename Stor<DT>::T* p, float* out) {
  if constexpr (DT == RECSA_BF16) {
    if constexpr (N == 8) {
      uint4 u = *reinterpret_cast<const uint4*>(p);
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else if constexpr (N == 4) {
      uint2 u = *reinterpret_cast<const uint2*>(p);
      out[0] = __uint_as_float(u.x << 16);
      out[1] = __uint_as_float(u.x & 0xFFFF0000u);
      out[2] = __uint_as_float(u.y << 16);
      out[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
      static_assert(N == 2, "vector width");
      uint32_t u = *reinterpret_cast<const uint32_t*>(p);
      out[0] = __uint_as_float(u << 16);
      out[1] = __uint_as_float(u & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      if constexpr (N >= 4) {
        float4 v = *reinterpret_cast<const float4*>(p + i);
        out[i] = v.x;
        out[i + 1] = v.y;
        out[i + 2] = v.z;
        out[i + 3] = v.w;
      }
    }
    if constexpr (N == 2) {
      float2 v = *reinterpret_cast<const float2*>(p);
      out[0] = v.x;
      out[1] = v.y;
    }
  }
}

// Store 8 floats as 8 consecutive storage elements (one 16-byte store for
// bf16, two for float32), each rounded to the storage dtype.
template <int DT>
__device__ __forceinline__ void store_vec8(typename Stor<DT>::T* p, const float* v) {
  if constexpr (DT == RECSA_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// ------------------------------------------------------------------- RoPE
// Rotate-half pair (x, y) by the angle whose (cos, sin) = (c, s):
// (x*c - y*s, x*s + y*c), each product and sum rounded to float32 separately
// (no fused multiply-add), so that the rounded operand is reproducible.
__device__ __forceinline__ void rope_pair(float x, float y, float c, float s,
                                          float& xo, float& yo) {
#pragma clang fp contract(off)
  const float xc = x * c;
  const float ys = y * s;
  const float xs = x * s;
  const float yc = y * c;
  xo = xc - ys;
  yo = xs + yc;
}

// Key half of the split RoPE for one stored row: the pairs (j, j + D/2) of
// `src`, rotated by the in-group offset c and rounded to the storage dtype,
// written to `dst`.  Pairs j0, j0 + jstep, ... are handled by the caller's
// thread.
template <int DT, int D>
__device__ __forceinline__ void rotate_key_row(const typename Stor<DT>::T* src,
                                               typename Stor<DT>::T* dst, int c,
                                               const float* __restrict__ rope, int j0,
                                               int jstep) {
  constexpr int H2 = D / 2;
  for (int j = j0; j < H2; j += jstep) {
    const float* rp = rope + (c * H2 + j) * 2;
    float xo, yo;
    rope_pair(Stor<DT>::load(src + j), Stor<DT>::load(src + j + H2), rp[0], rp[1], xo, yo);
    Stor<DT>::store(dst + j, xo);
    Stor<DT>::store(dst + j + H2, yo);
  }
}

// ------------------------------------------------------------- reductions
// Wave-wide reductions and scans with DPP row operations (plain VALU moves,
// no LDS crossbar): quad permutes and row rotates/shifts within each 16-lane
// row, then the row broadcasts of lanes 15 and 31 carry row results to the
// following rows; lane 63 ends with the total, which readlane broadcasts.
namespace dpp {
constexpr int kXor1 = 0xB1;                    // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;                    // quad_perm [2,3,0,1]
constexpr int kRor4 = 0x124, kRor8 = 0x128, kRor12 = 0x12C;   // row_ror:4, :8, :12
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;   // row_shr:n
constexpr int kBcast15 = 0x142, kBcast31 = 0x143;
}  // namespace dpp

// src moved by the DPP pattern CTRL; lanes whose source is outside the
// pattern, or whose row is not in ROWS, get `old`.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_mov(int old, int src) {
  return __builtin_amdgcn_update_dpp(old, src, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_movf(float old, float src) {
  return __int_as_float(dpp_mov<CTRL, ROWS>(__float_as_int(old), __float_as_int(src)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_movf<dpp::kXor1>(0.f, v);
  v += dpp_movf<dpp::kXor2>(0.f, v);
  v += dpp_movf<dpp::kRor4>(0.f, v);
  v += dpp_movf<dpp::kRor8>(0.f, v);
  v += dpp_movf<dpp::kBcast15, 0xA>(0.f, v);
  v += dpp_movf<dpp::kBcast31, 0xC>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_movf<dpp::kXor1>(v, v));
  v = fmaxf(v, dpp_movf<dpp::kXor2>(v, v));
  v = fmaxf(v, dpp_movf<dpp::kRor4>(v, v));
  v = fmaxf(v, dpp_movf<dpp::kRor8>(v, v));
  v = fmaxf(v, dpp_movf<dpp::kBcast15, 0xA>(v, v));
  v = fmaxf(v, dpp_movf<dpp::kBcast31, 0xC>(v, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// Sum of a value over the four 16-lane rows of the wave, in every lane:
// (x[l & ~16] + x[l | 16]) from v_permlane16_swap, then the same across the
// two 32-lane halves from v_permlane32_swap -- the additions of the
// xor-16 / xor-32 butterfly, in the same order.
__device__ __forceinline__ float row_sum4(float x) {
  const uint32_t xb = __float_as_uint(x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(xb, xb, false, false);
  const float y = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  const uint32_t yb = __float_as_uint(y);
  const auto p32 = __builtin_amdgcn_permlane32_swap(yb, yb, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

// Sum over each aligned quad of lanes (the result in all four lanes).
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_movf<dpp::kXor1>(0.f, v);
  v += dpp_movf<dpp::kXor2>(0.f, v);
  return v;
}

// Inclusive prefix sum over the 64 lanes (lane order).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_mov<dpp::kShr1>(0, v);
  v += dpp_mov<dpp::kShr2>(0, v);
  v += dpp_mov<dpp::kShr4>(0, v);
  v += dpp_mov<dpp::kShr8>(0, v);
  v += dpp_mov<dpp::kBcast15, 0xA>(0, v);
  v += dpp_mov<dpp::kBcast31, 0xC>(0, v);
  return v;
}

// Exclusive prefix sum over a 256-thread block; `red` is LDS of >= 4 ints.
// Returns the exclusive prefix and writes the block total to *total.
__device__ __forceinline__ int block_excl_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x >> 6;
  int inc = wave_incl_scan(v);
  if (lane == kWave - 1) red[wid] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kBlock / kWave; ++w) {
    int x = red[w];
    off += (w < wid) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// --------------------------------------------------------- list geometry
// Per (query, KV head, level l) view of the candidate list A^(l) of Eq. 3:
// A^(l) is the concatenation, in ascending node order, of the children of the
// selected nodes of level l+1, clipped at the current node a_l; at the top
// level it is [0 .. a_top].  Position p = C*r + c holds node C*S[r] + c.
struct ListView {
  int len;              // |A^(l)|
  int64_t cur;          // current node a_l
  const int32_t* up;    // S^(l+1) (ascending), nullptr at the top level
  __device__ __forceinline__ int64_t node(int p) const {
    return up ? static_cast<int64_t>(kC) * up[p / kC] + (p % kC) : static_cast<int64_t>(p);
  }
};

// Build the list view of level l.  sel/cnt point at this (query, head)'s
// selection arrays ([n_sel][k] and [n_sel]); top = n_levels - 1.
// When the level above holds the full prefix [0 .. a_{l+1}] with at most k
// nodes (always true at and above the top), it is fully selected and A^(l)
// is the full prefix [0 .. a_l]: no stored selection is read.
__device__ __forceinline__ ListView list_view(int64_t t, int l, int top, int k,
                                              const int32_t* sel, const int32_t* cnt) {
  ListView v;
  v.cur = t >> (4 * l);
  if (l >= top || (t >> (4 * (l + 1))) + 1 <= k) {
    v.len = static_cast<int>(v.cur) + 1;
    v.up = nullptr;
  } else {
    const int c_up = cnt[l];                    // |S^(l+1)| sits in slot l
    v.len = kC * (c_up - 1) + static_cast<int>(v.cur % kC) + 1;
    v.up = sel + static_cast<int64_t>(l) * k;
  }
  return v;
}

}  // namespace recsa
