// Eight RoPE pairs at a time, for kernels that rotate whole storage rows by
// a table row (the rotate-half pairs (j, j + d/2) and the fp32 rotation of
// picx.dev Key Theoretical Insight, as rope_pair evaluates it).
#pragma once

#include "recsa_common.hpp"

namespace recsa {

// Pairs (j, j + D/2), j in [j0, j0 + 8), of one storage row rotated by the
// table row `rrow` ([D/2][cos, sin] float32, 16-byte aligned): outputs xo
// (dims j) and yo (dims j + D/2).  j0 is a multiple of 8.
template <int DT, int D>
__device__ __forceinline__ void rotate8_pairs(const typename Stor<DT>::T* row, int j0,
                                              const float* __restrict__ rrow, float* xo,
                                              float* yo) {
  float x[8], y[8];
  load_vec<DT, 8>(row + j0, x);
  load_vec<DT, 8>(row + D / 2 + j0, y);
  float cs[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(rrow + 2 * j0 + 4 * i);
    cs[4 * i] = v.x;
    cs[4 * i + 1] = v.y;
    cs[4 * i + 2] = v.z;
    cs[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) rope_pair(x[e], y[e], cs[2 * e], cs[2 * e + 1], xo[e], yo[e]);
}

}  // namespace recsa
