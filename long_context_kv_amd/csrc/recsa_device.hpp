// Device building blocks shared by the selection / attention kernels:
// candidate-group logits with split candidate-local RoPE, query rotation,
// block reductions for any block size, the workgroup top-(k-1) selection and
// the per-group barrier used by the fused decode kernel.
#pragma once

#include "recsa_common.hpp"
#include "recsa_mfma.hpp"

namespace recsa {

// ------------------------------------------------------------------------
// Logits of the 16 rows of one list group against G rotated query heads.
// Lane = (row c = lane/4, quarter s = lane%4); each lane holds 2*E pairs of
// its row (as raw storage words) and dots them with the group's rotated
// query (LDS, float).  The rows are normally the stored rotated keys Kr,
// which already hold the key half of the split RoPE; with ROT the rows are
// raw keys, rotated here by the in-group offset c and rounded to the storage
// dtype (the same value Kr would hold).  The four quarter lanes of a row are
// summed, so every lane of row c ends with the G logits of that row.  Only
// rows in [row_lo, nvalid) are read; the others give 0.  Loading and
// computing are separate steps so a caller can issue the loads early.
// Two-term bf16 dot product accumulated in float32: the operands are the
// rounded (bf16) halves of the split RoPE, so every product is exact.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}

template <int DT, int D>
struct KRows {
  static constexpr int E = D / 16;
  static constexpr int WPC = DT == RECSA_BF16 ? E / 2 : E;   // 32-bit words per chunk
  uint32_t xr[2][WPC], yr[2][WPC];
};

template <int DT, int D>
__device__ __forceinline__ void group_load_k(const typename Stor<DT>::T* __restrict__ rows,
                                             int row_lo, int nvalid, KRows<DT, D>& kr) {
  constexpr int E = D / 16, QD = D / 4, H2 = D / 2, WPC = KRows<DT, D>::WPC;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane >> 2, s = lane & 3;
  if (c >= row_lo && c < nvalid) {
    const typename Stor<DT>::T* row = rows + static_cast<int64_t>(c) * D;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int base = hh * QD + s * E;
      const uint32_t* px = reinterpret_cast<const uint32_t*>(row + base);
      const uint32_t* py = reinterpret_cast<const uint32_t*>(row + H2 + base);
      if constexpr (WPC % 4 == 0) {
#pragma unroll
        for (int i = 0; i < WPC; i += 4) {
          const uint4 a = *reinterpret_cast<const uint4*>(px + i);
          const uint4 b = *reinterpret_cast<const uint4*>(py + i);
          kr.xr[hh][i] = a.x; kr.xr[hh][i + 1] = a.y; kr.xr[hh][i + 2] = a.z; kr.xr[hh][i + 3] = a.w;
          kr.yr[hh][i] = b.x; kr.yr[hh][i + 1] = b.y; kr.yr[hh][i + 2] = b.z; kr.yr[hh][i + 3] = b.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < WPC; ++i) {
          kr.xr[hh][i] = px[i];
          kr.yr[hh][i] = py[i];
        }
      }
    }
  } else {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < WPC; ++i) kr.xr[hh][i] = kr.yr[hh][i] = 0u;
  }
}

template <int DT, int D, int G, bool ROT = false>
__device__ __forceinline__ void group_logits_from(const KRows<DT, D>& kr, int row_lo, int nvalid,
                                                  const float* qt, const float* __restrict__ rope,
                                                  float* lg) {
  constexpr int E = D / 16, QD = D / 4, H2 = D / 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane >> 2, s = lane & 3;
  float acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.f;
  if (c >= row_lo && c < nvalid) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      // keep the two halves' LDS reads from being hoisted together
      __builtin_amdgcn_sched_barrier(0);
      const int base = hh * QD + s * E;
      const float* rp = rope + (c * H2 + base) * 2;
      if constexpr (DT == RECSA_BF16) {
        // packed words: dims (base + 2i, base + 2i + 1) of each half
        constexpr int WPC = E / 2;
        uint32_t kx[WPC], ky[WPC];
#pragma unroll
        for (int i = 0; i < WPC; ++i) {
          kx[i] = kr.xr[hh][i];
          ky[i] = kr.yr[hh][i];
        }
        if constexpr (ROT) {
#pragma unroll
          for (int i = 0; i < WPC; ++i) {
            float x0, y0, x1, y1;
            rope_pair(__uint_as_float(kx[i] << 16), __uint_as_float(ky[i] << 16), rp[4 * i],
                      rp[4 * i + 1], x0, y0);
            rope_pair(__uint_as_float(kx[i] & 0xFFFF0000u), __uint_as_float(ky[i] & 0xFFFF0000u),
                      rp[4 * i + 2], rp[4 * i + 3], x1, y1);
            kx[i] = pack_bf16x2(x0, x1);
            ky[i] = pack_bf16x2(y0, y1);
          }
        }
        const uint32_t* qw = reinterpret_cast<const uint32_t*>(qt);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint32_t* qx = qw + g * (D / 2) + base / 2;
          const uint32_t* qy = qw + g * (D / 2) + H2 / 2 + base / 2;
#pragma unroll
          for (int i = 0; i < WPC; ++i) {
            acc[g] = dot2_bf16(kx[i], qx[i], acc[g]);
            acc[g] = dot2_bf16(ky[i], qy[i], acc[g]);
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < E; ++m) {
          const float x = __uint_as_float(kr.xr[hh][m]);
          const float y = __uint_as_float(kr.yr[hh][m]);
          float xo = x, yo = y;
          if constexpr (ROT) rope_pair(x, y, rp[2 * m], rp[2 * m + 1], xo, yo);
#pragma unroll
          for (int g = 0; g < G; ++g)
            acc[g] += qt[g * D + base + m] * xo + qt[g * D + H2 + base + m] * yo;
        }
      }
    }
  }
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
#pragma unroll
  for (int g = 0; g < G; ++g) {
    lg[g] = quad_sum(acc[g]) * scale;
  }
}

// group_logits_from on rows that are either the stored rotated keys Kr
// (rot false) or raw keys rotated here (rot true: the tree keeps no Kr);
// both give the same bits.
template <int DT, int D, int G>
__device__ __forceinline__ void group_logits_any(bool rot, const KRows<DT, D>& kr, int row_lo,
                                                 int nvalid, const float* qt,
                                                 const float* __restrict__ rope, float* lg) {
  if (rot)
    group_logits_from<DT, D, G, true>(kr, row_lo, nvalid, qt, rope, lg);
  else
    group_logits_from<DT, D, G, false>(kr, row_lo, nvalid, qt, rope, lg);
}

// Rotate the G query heads by phi and round (one wave): qt = rnd(R(phi) q),
// the query half of the split RoPE.  Layout of qt: float [G][D] for fp32
// storage; for bf16 storage the rounded values are packed two per 32-bit
// word, [G][D/2] words (dims 2i, 2i+1 in word i, low half first), ready for
// the packed bf16 dot products.
// The (cos, sin) entries of table row phi that this lane's share of the
// query rotation needs, loaded ahead of the rotation.
template <int DT, int D, int G>
struct QRope {
  static constexpr int H2 = D / 2;
  static constexpr int ITEMS = DT == RECSA_BF16 ? G * H2 / 2 : G * H2;   // per wave
  static constexpr int PER_LANE = (ITEMS + kWave - 1) / kWave;
  float4 cs[PER_LANE];      // bf16: two pairs (cos, sin, cos, sin); fp32: (cos, sin, -, -)
};

template <int DT, int D, int G>
__device__ __forceinline__ void load_query_rope(int phi, const float* __restrict__ rope,
                                                QRope<DT, D, G>& r) {
  using Q = QRope<DT, D, G>;
  constexpr int H2 = D / 2;
  const int lane = threadIdx.x & (kWave - 1);
  const float* rrow = rope + static_cast<int64_t>(phi) * H2 * 2;
#pragma unroll
  for (int u = 0; u < Q::PER_LANE; ++u) {
    const int idx = lane + u * kWave;
    if (idx < Q::ITEMS) {
      if constexpr (DT == RECSA_BF16) {
        const int j = 2 * (idx % (H2 / 2));
        r.cs[u] = *reinterpret_cast<const float4*>(rrow + 2 * j);
      } else {
        const int j = idx % H2;
        const float2 v = *reinterpret_cast<const float2*>(rrow + 2 * j);
        r.cs[u] = make_float4(v.x, v.y, 0.f, 0.f);
      }
    }
  }
}

// The rotation itself from preloaded table entries: rnd(R(phi) q) of the
// G query heads into qt (LDS).
template <int DT, int D, int G>
__device__ __forceinline__ void rotate_query_from(const float* qs, float* qt,
                                                  const QRope<DT, D, G>& r) {
  using Q = QRope<DT, D, G>;
  constexpr int H2 = D / 2;
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int u = 0; u < Q::PER_LANE; ++u) {
    const int idx = lane + u * kWave;
    if (idx >= Q::ITEMS) continue;
    const float4 cs = r.cs[u];
    if constexpr (DT == RECSA_BF16) {
      uint32_t* qw = reinterpret_cast<uint32_t*>(qt);
      const int g = idx / (H2 / 2), j = 2 * (idx % (H2 / 2));
      float x0, y0, x1, y1;
      rope_pair(qs[g * D + j], qs[g * D + j + H2], cs.x, cs.y, x0, y0);
      rope_pair(qs[g * D + j + 1], qs[g * D + j + 1 + H2], cs.z, cs.w, x1, y1);
      qw[g * (D / 2) + j / 2] = pack_bf16x2(x0, x1);
      qw[g * (D / 2) + H2 / 2 + j / 2] = pack_bf16x2(y0, y1);
    } else {
      const int g = idx / H2, j = idx % H2;
      float xo, yo;
      rope_pair(qs[g * D + j], qs[g * D + j + H2], cs.x, cs.y, xo, yo);
      qt[g * D + j] = xo;
      qt[g * D + j + H2] = yo;
    }
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int DT, int D, int G, int NT>
__device__ __forceinline__ void load_query_rows(const void* q, int64_t row0, float* qs) {
  using T = typename Stor<DT>::T;
  const T* src = static_cast<const T*>(q) + row0 * D;
  for (int i = threadIdx.x; i < G * D; i += NT) qs[i] = Stor<DT>::load(src + i);
}

// ------------------------------------------------------------ reductions
// Block-wide reductions / scans for NT threads; `red` is LDS of NT/64 slots.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  constexpr int NW = NT / kWave;
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, red[w]);
  return r;
}

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  constexpr int NW = NT / kWave;
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) r += red[w];
  return r;
}

template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t v) {
  auto op = [](uint32_t a, int b) {
    return MAX ? max(a, static_cast<uint32_t>(b)) : min(a, static_cast<uint32_t>(b));
  };
  int x = static_cast<int>(v);
  v = op(v, dpp_mov<dpp::kXor1>(x, x));
  x = static_cast<int>(v);
  v = op(v, dpp_mov<dpp::kXor2>(x, x));
  x = static_cast<int>(v);
  v = op(v, dpp_mov<dpp::kRor4>(x, x));
  x = static_cast<int>(v);
  v = op(v, dpp_mov<dpp::kRor8>(x, x));
  x = static_cast<int>(v);
  v = op(v, dpp_mov<dpp::kBcast15, 0xA>(x, x));
  x = static_cast<int>(v);
  v = op(v, dpp_mov<dpp::kBcast31, 0xC>(x, x));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), kWave - 1));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_minmax_u32<false>(v); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_minmax_u32<true>(v); }

// Exclusive prefix sum over NT threads in thread order; total in *total.
template <int NT>
__device__ __forceinline__ int block_scan_excl(int v, int* red, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  __syncthreads();
  if (lane == kWave - 1) red[wid] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = red[w];
    off += (w < wid) ? x : 0;
    tot += x;
  }
  *total = tot;
  return off + inc - v;
}

// The same scan for a buffer no thread still reads (one used once per
// call): no barrier before its write.
template <int NT>
__device__ __forceinline__ int block_scan_excl_fresh(int v, int* red, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == kWave - 1) red[wid] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = red[w];
    off += (w < wid) ? x : 0;
    tot += x;
  }
  *total = tot;
  return off + inc - v;
}

// --------------------------------------------------------------- top-k
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;

constexpr int kSmallBin = 64;
constexpr float kLog2e = 1.44269504088896341f;

struct TopkSmem {
  int hist[kHistBins];
  uint32_t small_key[kSmallBin];
  int small_pos[kSmallBin];
  int small_rank[kSmallBin];   // keys of the boundary bin ranked above each
  int s_nsmall;
  float redg[kMaxG][16];      // per wave: softmax max of each head
  float reds[kMaxG][16];      // per wave: softmax normaliser of each head
  int redi[16];               // equal-key ranks
  int redt[16];               // take ranks
  int redb[2][16];            // radix bin totals per wave, by pass parity
  uint32_t redu[2][16];       // key range
  int s_bin, s_need, s_full;
};

// Selection at one scored level for one (query, KV head), by the whole
// workgroup (NT threads; thread i owns list positions [i*PPT, (i+1)*PPT)).
//   lgs    : logits [G][CK] of the n = |A|-1 non-current candidates
//   imp    : optional importance output [CK]
// Writes S^(l) (k-1 kept candidates in ascending order, then the current
// node), |S| = k, and the bitmap of kept list positions.
// Importance I_p = (1/G) sum_g softmax_p(s_g) is ranked through its float
// bits (I >= 0, so the bits order like the values); the (k-1)-th largest is
// found by 11-bit radix passes starting at the highest bit where the keys
// differ, and ties at the threshold go to the lower list position (= the
// lower node index, the list being in ascending node order).
// CKM: the list-size class (C*k <= CKM), so thread i owns PPT = CKM/NT
// positions; PPT divides C, so each thread's vector loads stay in its row.
template <int G, int NT, int CKM>
__device__ __attribute__((always_inline)) void wg_topk_cls(const float* __restrict__ lgs, int n, int k, int CK, const ListView& lv,
                            int32_t* out_sel, int32_t* out_cnt, uint32_t* bm, float* imp,
                            TopkSmem& sm) {
  static_assert(CKM <= kMaxCK && kC % (CKM / NT) == 0, "list-size class");
  constexpr int PPT = CKM / NT;
  const int tid = threadIdx.x;
  const int p0 = tid * PPT;
  constexpr int NW = NT / kWave;
  const int lane = tid & (kWave - 1), wid = tid >> 6;
  float e[G][PPT];
  float I[PPT];
  // the first radix pass's bins and the small-bin state start at zero
  // (ordered before their first use by the exchanges below)
  for (int b = tid; b < kHistBins; b += NT) sm.hist[b] = 0;
  for (int b = tid; b < kSmallBin; b += NT) sm.small_rank[b] = 0;
  if (tid == 0) sm.s_nsmall = 0;
  // ---- all logits first (one memory round trip), then per-head max and
  // normaliser with one block exchange for all heads
  // (each thread's PPT positions are contiguous and 16-byte aligned; the
  // logits row holds CK floats, so the vector loads stay inside it)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* src = lgs + static_cast<int64_t>(g) * CK + p0;
    if (p0 < n) {
#pragma unroll
      for (int i = 0; i < PPT; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + i);
        e[g][i] = v.x; e[g][i + 1] = v.y; e[g][i + 2] = v.z; e[g][i + 3] = v.w;
      }
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) if (p0 + i >= n) e[g][i] = -INFINITY;
  }
  {
    // per head: the max (one exchange), then the normaliser (a second
    // exchange on its own buffer, so neither needs a barrier before it)
    float M[G], Z[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < PPT; ++i) m = fmaxf(m, e[g][i]);
      M[g] = wave_max(m);
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) sm.redg[g][wid] = M[g];
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = sm.redg[g][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) m = fmaxf(m, sm.redg[g][w]);
      // exp(x - m) = 2^(x log2 e - m log2 e): one multiply-add and v_exp_f32
      // per entry; positions past the list hold -inf and give 0 (m is a
      // real logit, the list being non-empty); the rounding of m log2 e
      // scales every entry of the head alike and cancels in the normaliser
      const float nml = -m * kLog2e;
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        e[g][i] = __builtin_amdgcn_exp2f(fmaf(e[g][i], kLog2e, nml));
        z += e[g][i];
      }
      Z[g] = wave_sum(z);
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) sm.reds[g][wid] = Z[g];
    }
    __syncthreads();
    // each head's weight 1/(G Z_g) (1/G is a power of two, so exact)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float z = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) z += sm.reds[g][w];
      Z[g] = (1.0f / z) * (1.0f / G);
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      float s = e[0][i] * Z[0];
#pragma unroll
      for (int g = 1; g < G; ++g) s = fmaf(e[g][i], Z[g], s);
      I[i] = s;
    }
  }
  uint32_t key[PPT];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    key[i] = __float_as_uint(I[i]);
    if (p0 + i < n) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  }
  if (imp) {
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (p0 + i < CK) imp[p0 + i] = (p0 + i < n) ? I[i] : 0.f;
  }
  const int need0 = k - 1;
  uint32_t prefix = 0, pmask = 0;
  int need = need0;
  bool whole_bin = false, small = false;
  uint32_t small_m = 0u;          // my positions in the ranked boundary bin
  int small_at = 0;               // the bin slot of the first of them
  if (need0 > 0) {
    // the keys' range: the passes start at the highest bit where they differ,
    // so the first pass's bins resolve the keys finely (coarse bins would
    // pile many keys onto a few LDS counters)
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    if ((tid & (kWave - 1)) == 0) {
      sm.redu[0][tid >> 6] = kmin;
      sm.redu[1][tid >> 6] = kmax;
    }
    __syncthreads();
    kmin = sm.redu[0][0];
    kmax = sm.redu[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      kmin = min(kmin, sm.redu[0][w]);
      kmax = max(kmax, sm.redu[1][w]);
    }
    // highest differing bit (-1 when all keys are equal) and the mask of the
    // bits above it, which every key shares; the 64-bit shift keeps every
    // count in [0, 32] defined
    const uint32_t diff = kmin ^ kmax;
    int hb = diff ? 31 - __clz(diff) : -1;
    const int hb0 = hb;
    pmask = static_cast<uint32_t>(0xFFFFFFFFull << (hb + 1));
    prefix = kmin & pmask;
    int pass = 0;
#pragma unroll 1
    for (; hb >= 0; ++pass) {
      const int lo = max(hb - (kHistBits - 1), 0);
      const int nb = hb - lo + 1;
      const uint32_t dmask = (1u << nb) - 1u;
      if (hb < hb0) {                                // later passes clear their own bins
        __syncthreads();                             // after every read of the last pass's
        for (int b = tid; b < (1 << nb); b += NT) sm.hist[b] = 0;
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < PPT; ++i)
        if (p0 + i < n && (key[i] & pmask) == prefix) atomicAdd(&sm.hist[(key[i] >> lo) & dmask], 1);
      __syncthreads();
      // suffix counts over bins: thread t owns bins [t*BPT, (t+1)*BPT);
      // the keys above my range are those of the later lanes of my wave
      // and of the later waves (per-wave totals, one exchange; the two
      // buffers alternate between passes, so none is still being read)
      const int nbins = 1 << nb;
      const int bpt = (nbins + NT - 1) / NT;
      const int b0 = tid * bpt;
      int local = 0;
      for (int b = b0; b < min(b0 + bpt, nbins); ++b) local += sm.hist[b];
      const int incl = wave_incl_scan(local);
      const int wtot = __builtin_amdgcn_readlane(incl, kWave - 1);
      int* redb = sm.redb[pass & 1];
      if (lane == 0) redb[wid] = wtot;
      __syncthreads();
      int above = wtot - incl;
#pragma unroll
      for (int w = 0; w < NW; ++w) above += (w > wid) ? redb[w] : 0;
      for (int b = min(b0 + bpt, nbins) - 1; b >= b0; --b) {
        const int h = sm.hist[b];
        if (above < need && need <= above + h) {
          sm.s_bin = b;
          sm.s_need = need - above;
          sm.s_full = (need - above) == h;
        }
        above += h;
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(sm.s_bin) << lo;
      pmask |= dmask << lo;
      need = sm.s_need;
      whole_bin = sm.s_full != 0;
      const int in_bin = sm.hist[sm.s_bin];
      if (whole_bin) break;
      if (lo > 0 && in_bin <= kSmallBin) {
        // few keys left in the boundary bin: rank them exactly (key
        // descending, then list position ascending).  Each wave reserves
        // slots for its bin keys with one LDS atomic (a wave prefix sum
        // places its lanes' keys), then every wave ranks all bin keys (key
        // q sits in lane q) against a stride of them and adds its counts
#pragma unroll
        for (int i = 0; i < PPT; ++i)
          small_m |= (p0 + i < n && (key[i] & pmask) == prefix) ? (1u << i) : 0u;
        const int c_in = __popc(small_m);
        const int c_inc = wave_incl_scan(c_in);
        const int c_wave = __builtin_amdgcn_readlane(c_inc, kWave - 1);
        if (c_wave > 0) {
          int wbase = 0;
          if (lane == kWave - 1) wbase = atomicAdd(&sm.s_nsmall, c_wave);
          small_at = __builtin_amdgcn_readlane(wbase, kWave - 1) + c_inc - c_in;
          int at = small_at;
#pragma unroll
          for (int i = 0; i < PPT; ++i) {
            if ((small_m >> i) & 1u) {
              sm.small_key[at] = key[i];
              sm.small_pos[at] = p0 + i;
              ++at;
            }
          }
        }
        __syncthreads();
        {
          const int m = __builtin_amdgcn_readfirstlane(sm.s_nsmall);
          const uint32_t ki = lane < m ? sm.small_key[lane] : 0u;
          const int pi = lane < m ? sm.small_pos[lane] : 0;
          int rank = 0;
          for (int q2 = __builtin_amdgcn_readfirstlane(wid); q2 < m; q2 += NW) {
            const uint32_t kq = static_cast<uint32_t>(
                __builtin_amdgcn_readlane(static_cast<int>(ki), q2));
            const int pq = __builtin_amdgcn_readlane(pi, q2);
            rank += (kq > ki || (kq == ki && pq < pi)) ? 1 : 0;
          }
          if (lane < m && rank > 0) atomicAdd(&sm.small_rank[lane], rank);
        }
        __syncthreads();
        small = true;
        break;
      }
      hb = lo - 1;
    }
  }
  // ---- keep: truncated key above the threshold prefix, or equal to it and
  // (whole bin kept, ranked in by the small-bin pass, or among the first
  // `need` equal ones by position).  Per-thread flags are bit masks over the
  // PPT positions (bit i = position p0 + i).
  static_assert(PPT < 32 && 32 % PPT == 0, "positions per thread");
  uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const bool valid = need0 > 0 && p0 + i < n;
    const uint32_t kt = key[i] & pmask;
    gtm |= (valid && kt > prefix) ? (1u << i) : 0u;
    eqm |= (valid && kt == prefix) ? (1u << i) : 0u;
  }
  int tot;
  // the equal keys' ranks by position matter only when the boundary bin is
  // neither kept whole nor ranked by the small-bin pass
  const int eq_rank =
      (small || whole_bin) ? 0 : block_scan_excl_fresh<NT>(__popc(eqm), sm.redi, &tot);
  uint32_t inm;
  if (small) {
    // my bin keys sit at slots small_at, small_at + 1, ... in position order
    inm = 0u;
    int at = small_at;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      if ((small_m >> i) & 1u) {
        inm |= (sm.small_rank[at] < need) ? (1u << i) : 0u;
        ++at;
      }
    }
  } else if (whole_bin) {
    inm = eqm;
  } else {
    inm = 0u;
    int room = need - eq_rank;          // equal keys still wanted, in position order
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const bool e = ((eqm >> i) & 1u) != 0u;
      inm |= (e && room > 0) ? (1u << i) : 0u;
      room -= e ? 1 : 0;
    }
  }
  const uint32_t takem = gtm | inm;
  int slot = block_scan_excl_fresh<NT>(__popc(takem), sm.redt, &tot);
  if (takem) {
    // a thread's positions lie in one 16-position group (PPT divides C), so
    // one parent lookup serves them all; only the kept ones are visited
    const int64_t node0 = lv.node(p0);
    uint32_t tm = takem;
    while (tm) {
      const int i = __builtin_ctz(tm);
      tm &= tm - 1u;
      if (slot < k - 1) out_sel[slot] = static_cast<int32_t>(node0 + i);
      ++slot;
    }
  }
  // the count is k-1 by construction; should it ever fall short, the
  // remaining slots still name a real node (the current one), never stale data
  for (int i = tot + tid; i < k - 1; i += NT) out_sel[i] = static_cast<int32_t>(lv.cur);
  uint32_t bits = takem << (p0 & 31);
  // PPT consecutive positions per thread: 32/PPT threads share one word
  constexpr int LPW = 32 / PPT;
  static_assert(LPW <= 8, "bit words are merged within 8-lane groups");
  if constexpr (LPW >= 2) bits |= static_cast<uint32_t>(dpp_mov<dpp::kXor1>(0, static_cast<int>(bits)));
  if constexpr (LPW >= 4) bits |= static_cast<uint32_t>(dpp_mov<dpp::kXor2>(0, static_cast<int>(bits)));
  // the quads' words: row_ror:12 brings lane l + 4 to lane l, so the writing
  // lane (l % 8 == 0) takes the other quad of its 8-lane group
  if constexpr (LPW >= 8) bits |= static_cast<uint32_t>(dpp_mov<dpp::kRor12>(0, static_cast<int>(bits)));
  if ((tid % LPW) == 0 && p0 < CK) bm[p0 / 32] = bits;
  if (tid == 0) {
    out_sel[k - 1] = static_cast<int32_t>(lv.cur);
    *out_cnt = k;
  }
}

// The selection for a list of n + 1 candidates.  With 256 threads (many
// lists at once, as in a prefill chunk, where the vector units bound it),
// lists of at most half the class's positions take the half-size class, so
// each thread ranks half as many positions and none runs the per-position
// steps on positions past the list's end; the output words past the half
// class's reach are cleared as the full class would clear them.  The choice
// depends on n and the thread count alone, so every caller with the same
// thread count ranks a list with the same arithmetic.  512-thread callers
// (decode) keep one class: a second inlined copy would double the fused
// decode's code.
template <int G, int NT, int CKM = 4096>
__device__ __attribute__((always_inline)) void wg_topk(const float* __restrict__ lgs, int n, int k, int CK, const ListView& lv,
                        int32_t* out_sel, int32_t* out_cnt, uint32_t* bm, float* imp,
                        TopkSmem& sm) {
  constexpr int HALF = CKM / 2;
  if constexpr (NT == 256 && CKM / NT >= 8) {
    if (n <= HALF) {
      wg_topk_cls<G, NT, HALF>(lgs, n, k, CK, lv, out_sel, out_cnt, bm, imp, sm);
      if (imp)
        for (int p = HALF + static_cast<int>(threadIdx.x); p < CK; p += NT) imp[p] = 0.f;
      for (int wd = HALF / 32 + static_cast<int>(threadIdx.x); wd < (CK + 31) / 32; wd += NT)
        bm[wd] = 0u;
      return;
    }
  }
  wg_topk_cls<G, NT, CKM>(lgs, n, k, CK, lv, out_sel, out_cnt, bm, imp, sm);
}

// Fill the selection of a level whose list has at most k candidates (all kept).
template <int NT>
__device__ __forceinline__ void wg_take_all(const ListView& lv, int k, int32_t* out_sel,
                                            int32_t* out_cnt, float* imp, int CK) {
  for (int p = threadIdx.x; p < k; p += NT)
    out_sel[p] = p < lv.len ? static_cast<int32_t>(lv.node(p)) : -1;
  if (threadIdx.x == 0) *out_cnt = lv.len;
  if (imp)
    for (int p = threadIdx.x; p < CK; p += NT) imp[p] = 0.f;
}

// ------------------------------------------------------------ attention
// Per-query bookkeeping of the entry set E (Eq. 4) as 16-position groups:
// level 0 contributes every candidate (exact tokens, logits computed here);
// a scored level l >= 1 contributes its non-current candidates, of which the
// selected ones are masked out (their logits come from the workspace).
// Every access uses a compile-time index (unrolled loops) so the arrays stay
// in registers.
struct EntryGroups {
  int first[RECSA_MAX_LEVELS + 1];   // first group of each level; first[n_sel] = total
  int tot;
  __device__ __forceinline__ int total() const { return tot; }
  // level of group gi and the group's index within its level
  __device__ __forceinline__ void locate(int gi, int& level, int& local) const {
    level = 0;
    int base = 0;
#pragma unroll
    for (int l = 1; l < RECSA_MAX_LEVELS; ++l) {
      if (gi >= first[l] && first[l] < tot) {
        level = l;
        base = first[l];
      }
    }
    local = gi - base;
  }
};

__device__ __forceinline__ EntryGroups entry_groups(int64_t t, const recsa_tree& tr, int n_sel,
                                                    const int32_t* sel, const int32_t* cnt) {
  EntryGroups eg;
  const int top = tr.n_levels - 1;
  int acc = 0;
#pragma unroll
  for (int l = 0; l < RECSA_MAX_LEVELS; ++l) {
    eg.first[l] = acc;
    if (l < n_sel) {
      const ListView lv = list_view(t, l, top, tr.k, sel, cnt);
      int n = 0;
      if (l == 0) n = lv.len;
      else if (lv.len > tr.k) n = lv.len - 1;
      acc += (n + kC - 1) / kC;
    }
  }
  eg.first[RECSA_MAX_LEVELS] = acc;
  eg.tot = acc;
  return eg;
}

template <int D, int G, int NT>
struct AttnSmem {
  alignas(16) float qt[NT / kWave][G * D];
  float ew[NT / kWave][kWave][G];  // a chunk's per-entry logits, then its weights
  float wm[NT / kWave][G];
  float wl[NT / kWave][G];
  float wacc[NT / kWave][G][D];
  float res_m[G], res_l[G];      // merged state; the merged sum is in wacc[0]
};

// Softmax state of a set of entries: running max m, normaliser l, sum acc.
template <int G, int DPL>
struct SoftState {
  float m[G], l[G], acc[G][DPL];
};

// A wave processes its entries in chunks of NG 16-entry groups, one entry
// per lane for the softmax.
template <int DT, int D, int NG_MAX>
struct ChunkShape {
  // P V: lane = (class c = lane / 16, block b = lane % 16) owns the DPB dims
  // [b*DPB, (b+1)*DPB) of the entries e = c, c+4, c+8, ... of a chunk (one
  // 16-byte load per bf16 row, two per fp32 row at d = 128); the four
  // classes' partial sums are added once, after the last chunk.
  static constexpr int DPB = D / kC;                               // dims per lane
  static constexpr int VWE = (DT == RECSA_BF16) ? DPB / 2 : DPB;   // value words per entry
  static constexpr int NG = VWE == 8 ? (NG_MAX < 2 ? NG_MAX : 2) : NG_MAX;   // groups per chunk
  static constexpr int NE = NG * kC;                               // entries per chunk
  static constexpr int EPL = NE / 4;                               // entries per lane
};

// Per-level array entry with a per-lane level (unrolled selects: no
// dynamic indexing of the argument struct).
__device__ __forceinline__ const void* level_ptr(void* const (&arr)[RECSA_MAX_LEVELS], int level) {
  const void* r = arr[0];
#pragma unroll
  for (int l = 1; l < RECSA_MAX_LEVELS; ++l)
    if (level == l) r = arr[l];
  return r;
}

// A 64-bit value of lane src_lane.  Row addresses are formed as a tree
// array (a kernel argument) plus such an offset: the compiler then knows the
// address is global memory and issues global loads; an address read whole
// from another lane would be a generic one, whose flat loads also count
// against the LDS wait counter and stall the LDS work behind them.
__device__ __forceinline__ int64_t lane_i64(int64_t v, int src_lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), src_lane);
  const uint32_t hi =
      __builtin_amdgcn_readlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32), src_lane);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// One chunk of the entry set -- its 16-entry groups [gfirst, gend), at most
// NG of them -- folded into this wave's softmax state (m, lsum, acc).  HAS0:
// the chunk may hold level-0 groups, whose key rows are loaded and whose
// logits are formed here; without it every group is a summary group of a
// scored level (value rows and stored logits only).  Per chunk the level-0
// key rows are issued first, then the value rows, so both are in flight
// during the query rotations.  If k_t/v_t are given they replace the tree
// rows of token t (decode append in the same launch).
template <int DT, int D, int G, int NT, int NG, bool HAS0, bool MF = false>
__device__ __forceinline__ void attn_chunk(const recsa_tree& tr, int64_t t, int64_t seq_head,
                                           const int32_t* sel, const int32_t* cnt,
                                           const EntryGroups& eg, int gfirst, int gend,
                                           const float* qs, const float* __restrict__ lg_slot,
                                           const uint32_t* __restrict__ bm_slot, int CK,
                                           const typename Stor<DT>::T* k_t,
                                           const typename Stor<DT>::T* v_t, bool raw0,
                                           const void* kbase0, float (&m)[G], float (&lsum)[G],
                                           float (&acc)[G][D / kC], AttnSmem<D, G, NT>& sm) {
  using T = typename Stor<DT>::T;
  constexpr int DPB = D / kC;                                      // dims per lane
  constexpr int VWE = (DT == RECSA_BF16) ? DPB / 2 : DPB;          // value words per entry
  constexpr int NE = NG * kC, EPL = NE / 4;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  const int c = lane >> 2, s = lane & 3;
  const int top = tr.n_levels - 1;
  const int bm_words = (CK + 31) / 32;
  // ---- this lane's entry: row lane % 16 of group ci*NG + lane / 16
  const int gi = gfirst + lane / kC;
  const bool in_group = lane < NE && gi < gend;
  int level = 0, local = 0;
  if (in_group) eg.locate(gi, level, local);
  const ListView lv = list_view(t, level, top, tr.k, sel, cnt);
  const int p = local * kC + (lane % kC);
  const int n_pos = level == 0 ? lv.len : lv.len - 1;
  const bool valid = in_group && p < n_pos;
  const int64_t rows_l = level_rows_dev(tr.L_cap, level);
  const int64_t node = valid ? lv.node(p) : 0;
  // per group (read from the group's first lane): level-0 groups get logits here
  const int grp_nvalid = in_group ? min(kC, n_pos - local * kC) : 0;

  // ---- level-0 key rows and query-rotation table rows of the chunk's
  // groups (issued before the value rows, which are needed only last)
  static_assert(!MF || DT == RECSA_BF16, "matrix-core logits take bf16 rows");
  KRows<DT, D> ka[NG];                 // vector-unit logits: rows split over lane quads
  MFrag<D> kf[NG];                     // matrix-core logits: the B operand (row = lane % 16)
  QRope<DT, D, G> rq[NG];
  bool is0[NG];
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    const int lead = gg * kC;
    is0[gg] = HAS0 &&
              __builtin_amdgcn_readlane(static_cast<int>(in_group && level == 0), lead) != 0;
    if (is0[gg]) {
      const int nv = __builtin_amdgcn_readlane(grp_nvalid, lead);
      const int len = __builtin_amdgcn_readlane(lv.len, lead);
      const int p0 = __builtin_amdgcn_readlane(local, lead) * kC;
      const T* krow0 = static_cast<const T*>(kbase0) + lane_i64((seq_head * rows_l + node) * D, lead);
      const int ovr = k_t ? len - 1 - p0 : -1;          // row of token t, if in this group
      if constexpr (MF) {
        // lane l loads row l % 16; token t's row comes raw from k_t (rotated
        // before use), the group's last row when it is there; rows past the
        // group's end re-read its last row (their logits are masked)
        const int r = lane & 15, hq = lane >> 4;
        const uint16_t* src = (r == ovr) ? reinterpret_cast<const uint16_t*>(k_t)
                                         : reinterpret_cast<const uint16_t*>(krow0) + min(r, nv - 1) * D;
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb)
          kf[gg].w[kb] = *reinterpret_cast<const uint4*>(src + 8 * hq + 32 * kb);
      } else {
        group_load_k<DT, D>(krow0, 0, (ovr >= 0 && ovr < kC) ? ovr : nv, ka[gg]);
      }
      const int p_q = len - 1;
      load_query_rope<DT, D, G>(kC * (p_q / kC - p0 / kC) + p_q % kC, tr.rope, rq[gg]);
    }
  }
  // ---- summary logits (levels >= 1: from scoring, minus the selected ones)
  // (the loads do not wait for the selection bitmap: it masks afterwards)
  float lg[G];
  uint32_t sel_word = 0u;
  const bool summ = valid && level >= 1;
  {
    const float* src = lg_slot + static_cast<int64_t>(level - 1) * G * CK + p;
    if (summ) {
      sel_word = bm_slot[(level - 1) * bm_words + (p >> 5)];
#pragma unroll
      for (int g = 0; g < G; ++g) lg[g] = src[static_cast<int64_t>(g) * CK];
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) lg[g] = -INFINITY;
    }
  }
  // ---- value rows: a group's entries are 16 consecutive rows (children
  // of one parent), one row offset per group read from its first lane;
  // this lane loads its DPB dims of rows c, c+4, c+8, c+12 of each group;
  // token t's row may come from v_t.  Rows past the group's end (and every
  // row of a group past the chunk's end, which reads the first level-0 row)
  // re-read a valid row: their weights are 0.
  uint32_t vraw[EPL][VWE];
  const int64_t voff = (seq_head * rows_l + node) * D;
  const int vcls = lane >> 4, vdim = (lane & 15) * DPB;
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    const int lead = gg * kC;
    const int nv = __builtin_amdgcn_readlane(grp_nvalid, lead);
    const bool g0 =
        HAS0 && __builtin_amdgcn_readlane(static_cast<int>(in_group && level == 0), lead) != 0;
    const int len = __builtin_amdgcn_readlane(lv.len, lead);
    const int p0 = __builtin_amdgcn_readlane(local, lead) * kC;
    const int own_r = (g0 && k_t) ? len - 1 - p0 : -1;
    const int glevel = __builtin_amdgcn_readlane(level, lead);
    const T* vb = static_cast<const T*>(level_ptr(tr.V, glevel)) + lane_i64(voff, lead) + vdim;
    const int rlast = max(nv, 1) - 1;
#pragma unroll
    for (int rr = 0; rr < kC / 4; ++rr) {
      const int r = 4 * rr + vcls;                       // row within the group
      const int slot = gg * (kC / 4) + rr;               // this lane's entry slot
      const T* vr = (own_r == r) ? v_t + vdim : vb + min(r, rlast) * D;
      if constexpr (VWE == 4) {
        const uint4 x = *reinterpret_cast<const uint4*>(vr);
        vraw[slot][0] = x.x; vraw[slot][1] = x.y; vraw[slot][2] = x.z; vraw[slot][3] = x.w;
      } else if constexpr (VWE == 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(vr);
        vraw[slot][0] = x.x; vraw[slot][1] = x.y;
      } else {
#pragma unroll
        for (int u = 0; u < VWE; u += 4) {
          const uint4 x = *reinterpret_cast<const uint4*>(vr + u);
          vraw[slot][u] = x.x; vraw[slot][u + 1] = x.y; vraw[slot][u + 2] = x.z; vraw[slot][u + 3] = x.w;
        }
      }
    }
  }
  // ---- level-0 logits: split RoPE, one query rotation per group
  bool any0 = false;
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    if (!is0[gg]) continue;
    any0 = true;
    const int lead = gg * kC;
    const int nv = __builtin_amdgcn_readlane(grp_nvalid, lead);
    const int len = __builtin_amdgcn_readlane(lv.len, lead);
    const int p0 = __builtin_amdgcn_readlane(local, lead) * kC;
    const int ovr = k_t ? len - 1 - p0 : -1;
    const bool split = ovr >= 0 && ovr < kC;
    rotate_query_from<DT, D, G>(qs, sm.qt[wid], rq[gg]);
    if constexpr (MF) {
      // raw rows take the key half of the split RoPE here (every row without
      // a rotated copy, else only token t's): the values Kr holds
      if (raw0 || (split && (lane & 15) == ovr)) rotate_key_frag<D>(kf[gg], tr.rope);
      wave_sync();
      MFrag<D> qf;
      query_frag_lds<D, G>(reinterpret_cast<const uint16_t*>(sm.qt[wid]), qf);
      const f32x4_t acc4 = mfma_logits<D>(qf, kf[gg]);
      // C layout: lane l holds heads 4 (l / 16) + i of entry l % 16
      const int col = lane & 15, rb = lane >> 4;
      const float scale = 1.0f / sqrtf(static_cast<float>(D));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = 4 * rb + i;
        if (g < G) sm.ew[wid][lead + col][g] = (col < nv) ? acc4[i] * scale : -INFINITY;
      }
      wave_sync();
      continue;
    }
    wave_sync();
    float lgv[G];
    if (split) {
      // row t is not in Kr yet (appended in the same launch): rotate it here
      KRows<DT, D> kb;
      group_load_k<DT, D>(k_t - static_cast<int64_t>(ovr) * D, ovr, ovr + 1, kb);
      float a[G], b[G];
      group_logits_any<DT, D, G>(raw0, ka[gg], 0, ovr, sm.qt[wid], tr.rope, a);
      group_logits_from<DT, D, G, true>(kb, ovr, ovr + 1, sm.qt[wid], tr.rope, b);
#pragma unroll
      for (int g = 0; g < G; ++g) lgv[g] = (c == ovr) ? b[g] : a[g];
    } else {
      group_logits_any<DT, D, G>(raw0, ka[gg], 0, nv, sm.qt[wid], tr.rope, lgv);
    }
    if (s == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) sm.ew[wid][lead + c][g] = (c < nv) ? lgv[g] : -INFINITY;
    }
    wave_sync();
  }
  if (summ && ((sel_word >> (p & 31)) & 1u)) {      // selected: not an entry of E
#pragma unroll
    for (int g = 0; g < G; ++g) lg[g] = -INFINITY;
  }
  if (any0 && valid && level == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) lg[g] = sm.ew[wid][lane][g];
  }
  wave_sync();
  // ---- online softmax over the chunk (entry per lane); sums stay per lane
  float pr[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mnew = fmaxf(m[g], wave_max(lg[g]));
    if (mnew == -INFINITY) {
      pr[g] = 0.f;
      continue;
    }
    const float sc = (m[g] == -INFINITY) ? 0.f : __expf(m[g] - mnew);
    pr[g] = (lg[g] == -INFINITY) ? 0.f : __expf(lg[g] - mnew);
    lsum[g] = lsum[g] * sc + pr[g];
#pragma unroll
    for (int u = 0; u < DPB; ++u) acc[g][u] *= sc;
    m[g] = mnew;
  }
#pragma unroll
  for (int g = 0; g < G; ++g) sm.ew[wid][lane][g] = pr[g];
  wave_sync();
  // ---- P V (this lane: its DPB dims of its entries); a chunk's groups past
  // gend hold no entries (a short last chunk skips their work)
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    if (gfirst + gg >= gend) break;
#pragma unroll
    for (int rr = 0; rr < kC / 4; ++rr) {
      const int slot = gg * (kC / 4) + rr;
      const int e = gg * kC + 4 * rr + vcls;
      float v[DPB];
#pragma unroll
      for (int u = 0; u < DPB; ++u) {
        if constexpr (DT == RECSA_BF16) {
          const uint32_t wv = vraw[slot][u / 2];
          v[u] = __uint_as_float((u & 1) ? (wv & 0xFFFF0000u) : (wv << 16));
        } else {
          v[u] = __uint_as_float(vraw[slot][u]);
        }
      }
      float wgt[G];
#pragma unroll
      for (int g = 0; g < G; ++g) wgt[g] = sm.ew[wid][e][g];
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int u = 0; u < DPB; ++u) acc[g][u] += wgt[g] * v[u];
      }
    }
  }
  wave_sync();
}

// Process the entry chunks g_lo, g_lo + g_step, ... of one (query, KV head)
// with the whole workgroup (its waves take every NW-th of those; no block
// barrier inside the loop), then merge the waves: on return sm.res_m,
// sm.res_l and sm.wacc[0] hold the workgroup's softmax state (valid after
// the trailing __syncthreads), or, given part_out, the merge writes that
// state there as a partial [G][kPartHead + D] (max, sum, -, -, d values per
// query head) and returns without the barrier.  Chunks of NG_MAX groups (at most 2 with
// 8 value words per entry) run over the groups in order; with SPLIT the
// level-0 groups (key and value rows) form chunks of that size and the
// summary groups (value rows only) chunks of up to 4, which hold as many
// registers, so that each wave's loads go out in fewer rounds; there the
// level-0 logits of bf16 rows are formed on the matrix cores (a group's 16
// rows against the G rotated query heads, v_mfma_f32_16x16x32_bf16).
template <int DT, int D, int G, int NT, int NG_MAX = 4, bool SPLIT = false>
__device__ void attn_groups(const recsa_tree& tr, int64_t t, int64_t seq_head, const int32_t* sel,
                            const int32_t* cnt, const EntryGroups& eg, int g_lo, int g_step,
                            const float* qs, const float* __restrict__ lg_slot,
                            const uint32_t* __restrict__ bm_slot, int CK,
                            const typename Stor<DT>::T* k_t, const typename Stor<DT>::T* v_t,
                            AttnSmem<D, G, NT>& sm, float* __restrict__ part_out = nullptr) {
  using CS = ChunkShape<DT, D, NG_MAX>;
  constexpr int DPB = CS::DPB, NG = CS::NG;
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  float m[G], lsum[G], acc[G][DPB];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    lsum[g] = 0.f;
#pragma unroll
    for (int u = 0; u < DPB; ++u) acc[g][u] = 0.f;
  }
  const int n_groups = eg.total();
  const int n_chunks = (n_groups + NG - 1) / NG;
  // level-0 key rows: the stored rotated copy, or raw rows rotated here
  const bool raw0 = tr.Kr[0] == nullptr;
  const void* kbase0 = raw0 ? tr.K[0] : tr.Kr[0];
#pragma unroll 1
  for (int ci = g_lo + wid * g_step;; ci += NW * g_step) {
    if constexpr (SPLIT) {
      using CSS = ChunkShape<DT, D, 4>;
      const int n0 = eg.first[1];                       // level-0 groups come first
      const int c0 = (n0 + NG - 1) / NG;
      if (ci >= c0 + (n_groups - n0 + CSS::NG - 1) / CSS::NG) break;
      if (ci < c0) {
        attn_chunk<DT, D, G, NT, NG, true, DT == RECSA_BF16>(
            tr, t, seq_head, sel, cnt, eg, ci * NG, min(ci * NG + NG, n0), qs, lg_slot, bm_slot,
            CK, k_t, v_t, raw0, kbase0, m, lsum, acc, sm);
      } else {
        const int g0 = n0 + (ci - c0) * CSS::NG;
        attn_chunk<DT, D, G, NT, CSS::NG, false>(tr, t, seq_head, sel, cnt, eg, g0,
                                                 min(g0 + CSS::NG, n_groups), qs, lg_slot,
                                                 bm_slot, CK, k_t, v_t, raw0, kbase0, m, lsum,
                                                 acc, sm);
      }
    } else {
      if (ci >= n_chunks) break;
      attn_chunk<DT, D, G, NT, NG, true>(tr, t, seq_head, sel, cnt, eg, ci * NG,
                                         min(ci * NG + NG, n_groups), qs, lg_slot, bm_slot, CK,
                                         k_t, v_t, raw0, kbase0, m, lsum, acc, sm);
    }
  }
  // the four lane classes (16-lane rows) hold partial sums of the same dims:
  // add them with the gfx950 lane swaps, which read lanes l & ~16 and l | 16,
  // then l & 31 and (l & 31) + 32 (every lane ends with the totals)
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int u = 0; u < DPB; ++u)
      acc[g][u] = row_sum4(acc[g][u]);
  }
  SoftState<G, DPB> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = m[g];
    st.l[g] = wave_sum(lsum[g]);
#pragma unroll
    for (int u = 0; u < DPB; ++u) st.acc[g][u] = acc[g][u];
  }
  // ---- merge the waves
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (lane == 0) {
      sm.wm[wid][g] = st.m[g];
      sm.wl[wid][g] = st.l[g];
    }
    if (lane < kC) {
#pragma unroll
      for (int u = 0; u < DPB; ++u) sm.wacc[wid][g][lane * DPB + u] = st.acc[g][u];
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.wm[w][g]);
    float l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w)
        if (sm.wm[w][g] != -INFINITY) l += __expf(sm.wm[w][g] - M) * sm.wl[w][g];
    }
    if (part_out) {
      part_out[g * (D + kPartHead)] = M;
      part_out[g * (D + kPartHead) + 1] = l;
    } else {
      sm.res_m[g] = M;
      sm.res_l[g] = l;
    }
  }
  // each (g, d) is read and then overwritten by exactly one thread
  for (int e = threadIdx.x; e < G * D; e += NT) {
    const int g = e / D, dd = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.wm[w][g]);
    float a = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = sm.wm[w][g];
        if (mw != -INFINITY) a += __expf(mw - M) * sm.wacc[w][g][dd];
      }
    }
    if (part_out)
      part_out[g * (D + kPartHead) + kPartHead + dd] = a;
    else
      sm.wacc[0][g][dd] = a;
  }
  if (!part_out) __syncthreads();
}

// Merge n_split partial softmax states [n_split][G][D+2] = (m, l, acc[D])
// into out [G][D].  Threads own (g, d) pairs and walk the splits with
// several loads in flight.
template <int D, int G, int NT>
__device__ __forceinline__ void merge_partials(const float* __restrict__ pp, int n_split,
                                               float* __restrict__ o) {
  const int stride = G * (D + kPartHead);
  for (int e = threadIdx.x; e < G * D; e += NT) {
    const int g = e / D, dd = e % D;
    float M = -INFINITY, a = 0.f, l = 0.f;
    for (int s0 = 0; s0 < n_split; s0 += 8) {
      float ms[8], ls[8], as[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = s0 + i < n_split;
        const float* q = pp + (s0 + i) * stride + g * (D + kPartHead);
        ms[i] = ok ? q[0] : -INFINITY;
        ls[i] = ok ? q[1] : 0.f;
        as[i] = ok ? q[kPartHead + dd] : 0.f;
      }
      float mb = M;
#pragma unroll
      for (int i = 0; i < 8; ++i) mb = fmaxf(mb, ms[i]);
      if (mb == -INFINITY) continue;
      const float sc = (M == -INFINITY) ? 0.f : __expf(M - mb);
      a *= sc;
      l *= sc;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float f = (ms[i] == -INFINITY) ? 0.f : __expf(ms[i] - mb);
        a += f * as[i];
        l += f * ls[i];
      }
      M = mb;
    }
    o[e] = a / l;
  }
}

}  // namespace recsa
