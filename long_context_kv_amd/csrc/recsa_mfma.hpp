// Selection logits on the gfx950 matrix cores (bf16 storage only): the
// logits of one 16-row candidate group -- the B operand, its rows are the
// output columns -- against up to 16 rotated query rows -- the A operand --
// with v_mfma_f32_16x16x32_bf16, D/32 k blocks accumulated in ascending
// order.  Every path that forms a selection logit (per-query scoring, the
// fused decode, the bucketed multi-query scoring) goes through
// mfma_logits, so a (query row, key row) pair gets the same float32 logit
// whichever kernel computes it and wherever the row sits in the tile.
//
// Lane layout of the instruction (checked on the device):
//   A: lane l holds row l%16, k = 8*(l/16) + [0, 8) of each 32-wide block
//   B: lane l holds column l%16, the same k
//   C: lane l holds rows 4*(l/16) + i, i = 0..3, of column l%16
// The operands are the two rounded halves of the split candidate-local
// RoPE (picx.dev, Key Theoretical Insight): rnd(R(phi) q) and the stored
// rotated key rows Kr = rnd(R(c) K); every bf16 product is exact in float32.
#pragma once

#include "recsa_common.hpp"

namespace recsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One lane's share of a 16 x D bf16 operand: 8 dims of each 32-wide block.
template <int D>
struct MFrag {
  static_assert(D % 64 == 0, "head dim");
  uint4 w[D / 32];
};

// B operand: rows [0, nrows) of a group of 16 consecutive stored rows; the
// other rows read as 0 (their logits are never stored).
template <int D>
__device__ __forceinline__ void load_key_frag(const uint16_t* __restrict__ rows, int nrows,
                                              MFrag<D>& f) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, h = lane >> 4;
  if (r < nrows) {
    const uint16_t* p = rows + static_cast<int64_t>(r) * D + 8 * h;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) f.w[kb] = *reinterpret_cast<const uint4*>(p + 32 * kb);
  } else {
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) f.w[kb] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// A operand from G rotated query heads already in LDS (bf16, [G][D] in
// natural dim order, 16-byte aligned): row m < G is head m, rows >= G are 0.
template <int D, int G>
__device__ __forceinline__ void query_frag_lds(const uint16_t* qt, MFrag<D>& f) {
  const int lane = threadIdx.x & (kWave - 1);
  const int m = lane & 15, h = lane >> 4;
  if (m < G) {
    const uint16_t* p = qt + m * D + 8 * h;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) f.w[kb] = *reinterpret_cast<const uint4*>(p + 32 * kb);
  } else {
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) f.w[kb] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// The (cos, sin) entries of table row phi for the pairs this lane rotates in
// rotate_frag: 8 pairs per block pair, loaded once and reused for every
// query head of the row.
template <int D>
struct RopeFrag {
  float4 cs[D / 64][4];
};

template <int D>
__device__ __forceinline__ void load_rope_frag(int phi, const float* __restrict__ rope,
                                               RopeFrag<D>& r) {
  constexpr int H2 = D / 2;
  const int h = (threadIdx.x & (kWave - 1)) >> 4;
  const float* rrow = rope + static_cast<int64_t>(phi) * H2 * 2;
#pragma unroll
  for (int kb = 0; kb < D / 64; ++kb)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      r.cs[kb][v] = *reinterpret_cast<const float4*>(rrow + 2 * (32 * kb + 8 * h) + 4 * v);
}

// A operand row of this lane: the bf16 query row qrow rotated with the
// table entries in r and rounded, rnd(R(phi) q) -- the values rotate_query_from
// produces.  The block pairs (kb, kb + D/64) hold dims j and j + D/2, the
// two members of a RoPE pair, so each lane rotates its own 8 pairs per
// block pair.
template <int D>
__device__ __forceinline__ void rotate_frag(const uint16_t* __restrict__ qrow,
                                            const RopeFrag<D>& r, MFrag<D>& f) {
  constexpr int H2 = D / 2, HKB = D / 64;
  const int h = (threadIdx.x & (kWave - 1)) >> 4;
  // every load of the row first (one memory round trip), then the rotations
  uint4 xws[HKB], yws[HKB];
#pragma unroll
  for (int kb = 0; kb < HKB; ++kb) {
    xws[kb] = *reinterpret_cast<const uint4*>(qrow + 32 * kb + 8 * h);
    yws[kb] = *reinterpret_cast<const uint4*>(qrow + H2 + 32 * kb + 8 * h);
  }
#pragma unroll
  for (int kb = 0; kb < HKB; ++kb) {
    const uint4 xw = xws[kb], yw = yws[kb];
    const uint32_t xa[4] = {xw.x, xw.y, xw.z, xw.w};
    const uint32_t ya[4] = {yw.x, yw.y, yw.z, yw.w};
    uint32_t xo[4], yo[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x0, y0, x1, y1;
      rope_pair(__uint_as_float(xa[v] << 16), __uint_as_float(ya[v] << 16), r.cs[kb][v].x,
                r.cs[kb][v].y, x0, y0);
      rope_pair(__uint_as_float(xa[v] & 0xFFFF0000u), __uint_as_float(ya[v] & 0xFFFF0000u),
                r.cs[kb][v].z, r.cs[kb][v].w, x1, y1);
      xo[v] = pack_bf16x2(x0, x1);
      yo[v] = pack_bf16x2(y0, y1);
    }
    f.w[kb] = make_uint4(xo[0], xo[1], xo[2], xo[3]);
    f.w[kb + HKB] = make_uint4(yo[0], yo[1], yo[2], yo[3]);
  }
}

// The key half of the split RoPE applied in registers to a B operand loaded
// from raw (unrotated) key rows: lane l holds row l%16 of a 16-row group
// aligned to a multiple of 16 nodes, so its in-group offset is l%16, and it
// rotates its own 8 pairs per block pair by that offset and rounds --
// rnd(R(c) K), the value the stored rotated rows Kr hold, bit for bit.
template <int D>
__device__ __forceinline__ void rotate_key_frag(MFrag<D>& f, const float* __restrict__ rope) {
  constexpr int HKB = D / 64;
  RopeFrag<D> r;
  load_rope_frag<D>(threadIdx.x & 15, rope, r);
#pragma unroll
  for (int kb = 0; kb < HKB; ++kb) {
    const uint32_t xa[4] = {f.w[kb].x, f.w[kb].y, f.w[kb].z, f.w[kb].w};
    const uint32_t ya[4] = {f.w[kb + HKB].x, f.w[kb + HKB].y, f.w[kb + HKB].z, f.w[kb + HKB].w};
    uint32_t xo[4], yo[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x0, y0, x1, y1;
      rope_pair(__uint_as_float(xa[v] << 16), __uint_as_float(ya[v] << 16), r.cs[kb][v].x,
                r.cs[kb][v].y, x0, y0);
      rope_pair(__uint_as_float(xa[v] & 0xFFFF0000u), __uint_as_float(ya[v] & 0xFFFF0000u),
                r.cs[kb][v].z, r.cs[kb][v].w, x1, y1);
      xo[v] = pack_bf16x2(x0, x1);
      yo[v] = pack_bf16x2(y0, y1);
    }
    f.w[kb] = make_uint4(xo[0], xo[1], xo[2], xo[3]);
    f.w[kb + HKB] = make_uint4(yo[0], yo[1], yo[2], yo[3]);
  }
}

// Split 8 float32 values into bf16 halves, hi = rnd(x) and lo = rnd(x - hi),
// packed two per word: hi + lo holds x to about 2^-17 relative, so that
// hi.hi + hi.lo + lo.hi on the matrix cores gives a float32-level product.
__device__ __forceinline__ void split_bf16x8(const float* x, uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint16_t a = f32_to_bf16_bits(x[2 * v]), b = f32_to_bf16_bits(x[2 * v + 1]);
    const float ra = x[2 * v] - bf16_bits_to_f32(a), rb = x[2 * v + 1] - bf16_bits_to_f32(b);
    h[v] = static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
    l[v] = pack_bf16x2(ra, rb);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// C = A B^T over the D dims, k blocks in ascending order (unscaled).
template <int D>
__device__ __forceinline__ f32x4_t mfma_logits(const MFrag<D>& a, const MFrag<D>& b) {
  f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.w[kb]),
                                                __builtin_bit_cast(bf16x8_t, b.w[kb]), c, 0, 0, 0);
  return c;
}

// Store the logits (times 1/sqrt(D)) of one tile whose A rows are the G
// query heads (row g = head g) and whose B rows are list positions p0 ..
// p0+15: head g is output row g, which lane 16*(g/4) + col holds as element
// g%4 (the C layout above); positions at or past p0 + nvalid are not stored.
template <int D, int G>
__device__ __forceinline__ void store_logit_tile(const f32x4_t& c, float* out, int CK, int p0,
                                                 int nvalid) {
  const int lane = threadIdx.x & (kWave - 1);
  const int col = lane & 15, rb = lane >> 4;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  if (col < nvalid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * rb + i;
      if (g < G) out[static_cast<int64_t>(g) * CK + p0 + col] = c[i] * scale;
    }
  }
}

}  // namespace recsa
