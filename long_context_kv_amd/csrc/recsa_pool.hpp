// Pooling of C=16 children into one tree node (picx.dev Tree Construction,
// Eq. 1 for values; Pooler Distillation, Eq. 5 for keys), for a tile of
// NODES consecutive nodes and a workgroup of NT threads.  Arithmetic is
// float32; the node is rounded once to the storage dtype when stored.
#pragma once

#include "recsa_common.hpp"
#include "recsa_mfma.hpp"

namespace recsa {

// ---------------------------------------------------------- pooling tile
// One workgroup pools NODES consecutive nodes of one (sequence, KV head).
// Phase 1 (one wave per node): children statistics, alpha, p, value mean.
// Phase 2/3 (all threads): the pooler MLP for the tile, weights streamed
// from L2 once per tile.  Phase 4: K = mu + g (p - mu) + sigma m.
// Phase 5: the rotated key rnd(R(c) K) of each node, c = node index mod C.
// With STATS set (the shift penalty of Eq. 7) nothing is stored: phases 4-5
// are replaced by the tile's sums of sigma*m (D values) and of ||mu||^2,
// written to stats[0 .. D]; vc, vo, ko and kro are not used.
// Wave totals of 16 per-lane values at once: a reduce-scatter over the lane
// bits (each step keeps half the values and adds the partner lane's other
// half), so lane l ends with the total of value l % 16; then every lane reads
// the 16 totals back.  About 60 instructions instead of 16 separate
// reductions; every exchange is a DPP move or a gfx950 lane swap (no LDS).
__device__ __forceinline__ void wave_sum16(float (&v)[16]) {
  const int lane = threadIdx.x & (kWave - 1);
  float a[8];
  {
    const bool hi = lane & 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float keep = hi ? v[2 * j + 1] : v[2 * j];
      const float send = hi ? v[2 * j] : v[2 * j + 1];
      a[j] = keep + dpp_movf<dpp::kXor1>(0.f, send);
    }
  }
  float b[4];                           // value 4 j + 2 bit1 + bit0 of the lane
  {
    const bool hi = lane & 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float keep = hi ? a[2 * j + 1] : a[2 * j];
      const float send = hi ? a[2 * j] : a[2 * j + 1];
      b[j] = keep + dpp_movf<dpp::kXor2>(0.f, send);
    }
  }
  float c2[2];
  {
    // lane l ^ 4 within the 16-lane row: row_ror:12 reads lane l + 4 (the
    // partner of the lanes with bit 2 clear), row_ror:4 lane l - 4
    const bool hi = lane & 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float keep = hi ? b[2 * j + 1] : b[2 * j];
      const float send = hi ? b[2 * j] : b[2 * j + 1];
      const float up = dpp_movf<dpp::kRor12>(0.f, send), down = dpp_movf<dpp::kRor4>(0.f, send);
      c2[j] = keep + (hi ? down : up);
    }
  }
  float t;
  {
    const bool hi = lane & 8;              // lane l ^ 8: row_ror:8 (its own inverse)
    const float keep = hi ? c2[1] : c2[0];
    const float send = hi ? c2[0] : c2[1];
    t = keep + dpp_movf<dpp::kRor8>(0.f, send);
  }
  t = row_sum4(t);
#pragma unroll
  for (int c = 0; c < 16; ++c)
    v[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), c));
}

template <int DT, int D, int NODES>
struct PoolSmem {
  // rows padded by 16 bytes, so the 16 rows of a matrix-core operand read
  // from LDS fall in different banks.  feat (the MLP input, 2D per node) is
  // dead once the MLP's first layer has read it, so the MLP output m (D per
  // node), and after it the stored node key, take the same rows: the tile
  // needs 8 KB less LDS, and four tiles fit a CU instead of three.
  union {
    float feat[NODES][2 * D + 4];
    float m[NODES][2 * D + 4];
  };
  float hid[NODES][256 + 4];
};
// The pooler MLP of a tile on the float32 matrix cores (bf16 trees): hid =
// SiLU(W1 feat + b1), then m = W2 hid, as [16 nodes] x [k] x [16 outputs]
// tiles of v_mfma_f32_16x16x4_f32 (float32 products and sums, like the vector
// path).  Per 16-wide k block, lane group h holds k = 16 kb + 4h .. 4h+3 of
// its row as one float4 and instruction s takes element s of it, for A and B
// alike.  Rows are nodes (rows at or past n_valid, or past NODES, read as 0;
// their outputs are not stored); the waves take the output tiles in turn.  A
// node's result does not depend on the tile's other rows, so a tile of one
// node (decode append) gives the bits a full tile gives.  Ends with a
// workgroup barrier.
template <int D, int NODES, int NT>
__device__ void pool_mlp_mfma(const recsa_pooler& P, int n_valid, float (*feat)[2 * D + 4],
                              float (*hid)[256 + 4], float (*mo)[2 * D + 4]) {
  constexpr int NWAVES = NT / kWave;
  constexpr int K1 = 2 * D;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  const int row = lane & 15, h = lane >> 4;
  const bool arow = row < NODES && row < n_valid;
  const int H = P.hidden;
  const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
  // ---- layer 1: output tiles of 16 hidden units, two per wave at a time
  // (two independent accumulation chains over the same A operand)
  for (int t = wid; t < H / 16; t += 2 * NWAVES) {
    const int t2 = t + NWAVES;
    const bool two = t2 < H / 16;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
    const float* wrow = P.W1 + static_cast<int64_t>(16 * t + row) * K1 + 4 * h;
    const float* wrow2 = two ? P.W1 + static_cast<int64_t>(16 * t2 + row) * K1 + 4 * h : wrow;
#pragma unroll 4
    for (int kb = 0; kb < K1 / 16; ++kb) {
      const float4 b = *reinterpret_cast<const float4*>(wrow + 16 * kb);
      const float4 b2 = *reinterpret_cast<const float4*>(wrow2 + 16 * kb);
      const float4 a = arow ? *reinterpret_cast<const float4*>(&feat[row][16 * kb + 4 * h]) : zero4;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b2.x, acc2, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b2.y, acc2, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b2.z, acc2, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b2.w, acc2, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q == 1 && !two) break;
      const int hu = 16 * (q ? t2 : t) + row;      // this lane's hidden unit
      const float bias = P.b1[hu];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 4 * h + i;
        if (n < NODES) {
          const float z = (q ? acc2[i] : acc[i]) + bias;
          hid[n][hu] = z / (1.0f + __expf(-z));
        }
      }
    }
  }
  __syncthreads();
  // ---- layer 2: output tiles of 16 key dims (k = the hidden units), two
  // per wave at a time
  for (int t = wid; t < D / 16; t += 2 * NWAVES) {
    const int t2 = t + NWAVES;
    const bool two = t2 < D / 16;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
    const float* wrow = P.W2 + static_cast<int64_t>(16 * t + row) * H + 4 * h;
    const float* wrow2 = two ? P.W2 + static_cast<int64_t>(16 * t2 + row) * H + 4 * h : wrow;
#pragma unroll 4
    for (int kb = 0; kb < H / 16; ++kb) {
      const float4 b = *reinterpret_cast<const float4*>(wrow + 16 * kb);
      const float4 b2 = *reinterpret_cast<const float4*>(wrow2 + 16 * kb);
      const float4 a = arow ? *reinterpret_cast<const float4*>(&hid[row][16 * kb + 4 * h]) : zero4;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b2.x, acc2, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b2.y, acc2, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b2.z, acc2, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b2.w, acc2, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q == 1 && !two) break;
      const int j = 16 * (q ? t2 : t) + row;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 4 * h + i;
        if (n < NODES) mo[n][j] = q ? acc2[i] : acc[i];
      }
    }
  }
  __syncthreads();
}


template <int DT, int D, int NODES, int NT, bool STATS = false>
__device__ void pool_tile(const typename Stor<DT>::T* __restrict__ kc,  // child K rows
                          const typename Stor<DT>::T* __restrict__ vc,  // child V rows
                          typename Stor<DT>::T* __restrict__ ko,        // node K rows
                          typename Stor<DT>::T* __restrict__ vo,        // node V rows
                          typename Stor<DT>::T* __restrict__ kro,       // rotated node K rows
                          int c0,                   // index mod C of the tile's first node
                          const float* __restrict__ rope,
                          int n_valid, const recsa_pooler& P,
                          PoolSmem<DT, D, NODES>& sm, float* __restrict__ stats = nullptr,
                          typename Stor<DT>::T* __restrict__ krc = nullptr) {
  using T = typename Stor<DT>::T;
  constexpr int DPL = D / kWave;                 // dims per lane (1 or 2)
  constexpr int NWAVES = NT / kWave;
  constexpr int NPW = (NODES + NWAVES - 1) / NWAVES;   // nodes per wave
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x >> 6;
  const int i0 = lane * DPL;

  float mu_r[NPW][DPL], p_r[NPW][DPL], sig_r[NPW], mu2_r[NPW];

  // ---- phase 1
#pragma unroll
  for (int nw = 0; nw < NPW; ++nw) {
    const int n = wid * NPW + nw;
    sig_r[nw] = 0.f;
    mu2_r[nw] = 0.f;
    if (n >= NODES || n >= n_valid) continue;
    float x[kC][DPL];
    float vs[DPL];
#pragma unroll
    for (int u = 0; u < DPL; ++u) vs[u] = 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const T* kr = kc + (static_cast<int64_t>(n) * kC + c) * D + i0;
      if constexpr (DPL == 2)
        load_vec<DT, 2>(kr, x[c]);
      else
        x[c][0] = Stor<DT>::load(kr);
      if constexpr (!STATS) {
        const T* vr = vc + (static_cast<int64_t>(n) * kC + c) * D + i0;
        if constexpr (DPL == 2) {
          float tmp[2];
          load_vec<DT, 2>(vr, tmp);
          vs[0] += tmp[0];
          vs[1] += tmp[1];
        } else {
          vs[0] += Stor<DT>::load(vr);
        }
      }
    }
    // the children's rotated key rows krc = rnd(R(c) K) (R13's key half; a
    // node's children sit at in-group offsets 0..15), while the rows are in
    // registers: dim j's RoPE partner j + D/2 is in lane l ^ 32 (same slot),
    // which v_permlane32_swap exchanges; both lanes form the pair with
    // rope_pair and keep their own member, so the bits equal the separate
    // rotation pass's
    if constexpr (!STATS) {
      if (krc) {
        constexpr int H2 = D / 2;
        const int jl = (lane & 31) * DPL;          // this lane pair's first dim below D/2
        const bool low = lane < 32;
#pragma unroll 4
        for (int c = 0; c < kC; ++c) {
          float cs[2 * DPL];
          if constexpr (DPL == 2) {
            const float4 r = *reinterpret_cast<const float4*>(rope + (c * H2 + jl) * 2);
            cs[0] = r.x; cs[1] = r.y; cs[2] = r.z; cs[3] = r.w;
          } else {
            const float2 r = *reinterpret_cast<const float2*>(rope + (c * H2 + jl) * 2);
            cs[0] = r.x; cs[1] = r.y;
          }
          float o[DPL];
#pragma unroll
          for (int u = 0; u < DPL; ++u) {
            const uint32_t xb = __float_as_uint(x[c][u]);
            const auto pr = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
            float xo, yo;
            rope_pair(__uint_as_float(pr[0]), __uint_as_float(pr[1]), cs[2 * u], cs[2 * u + 1], xo,
                      yo);
            o[u] = low ? xo : yo;
          }
          T* dst = krc + (static_cast<int64_t>(n) * kC + c) * D + i0;
          if constexpr (DPL == 2 && DT == RECSA_BF16) {
            *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(o[0], o[1]);
          } else {
#pragma unroll
            for (int u = 0; u < DPL; ++u) Stor<DT>::store(dst + u, o[u]);
          }
        }
      }
    }
    // value mean (Eq. 1)
    if constexpr (!STATS) {
#pragma unroll
      for (int u = 0; u < DPL; ++u)
        Stor<DT>::store(vo + static_cast<int64_t>(n) * D + i0 + u, vs[u] * (1.0f / kC));
    }
    // mu, sigma, rho
    float mu[DPL];
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kC; ++c) s += x[c][u];
      mu[u] = s * (1.0f / kC);
    }
    float sq = 0.f, mq = 0.f;
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        const float dv = x[c][u] - mu[u];
        sq += dv * dv;
      }
      mq += mu[u] * mu[u];
    }
    sq = wave_sum(sq);
    mq = wave_sum(mq);
    const float sigma = sqrtf(sq / static_cast<float>(kC * D) + P.eps);
    const float rho = sqrtf(mq / static_cast<float>(D) + P.eps);
    // alpha_c = softmax_c(tau * w.(x_c - mu) / sigma)
    float w[DPL];
#pragma unroll
    for (int u = 0; u < DPL; ++u) w[u] = P.w[i0 + u];
    float a[kC];
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      float s = 0.f;
#pragma unroll
      for (int u = 0; u < DPL; ++u) s += w[u] * (x[c][u] - mu[u]);
      a[c] = s;
    }
    static_assert(kC == 16, "children per node");
    wave_sum16(a);
    const float scale = P.tau / sigma;
    float amax = -INFINITY;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      a[c] *= scale;
      amax = fmaxf(amax, a[c]);
    }
    float asum = 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      a[c] = __expf(a[c] - amax);
      asum += a[c];
    }
    const float inv = 1.0f / asum;
    float p[DPL];
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kC; ++c) s += a[c] * x[c][u];
      p[u] = s * inv;
    }
    const float inv_rho = 1.0f / rho, inv_sig = 1.0f / sigma;
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      sm.feat[n][i0 + u] = mu[u] * inv_rho;
      sm.feat[n][D + i0 + u] = (p[u] - mu[u]) * inv_sig;
      mu_r[nw][u] = mu[u];
      p_r[nw][u] = p[u];
    }
    sig_r[nw] = sigma;
    mu2_r[nw] = mq;
  }
  __syncthreads();

  if constexpr (DT == RECSA_BF16) {
    pool_mlp_mfma<D, NODES, NT>(P, n_valid, sm.feat, sm.hid, sm.m);
  } else {
  // ---- phase 2: hid = SiLU(W1 feat + b1)
  // nodes per thread: 8 with 256 threads, 4 with 512 (one item per thread
  // for 16 nodes and 128 hidden units); the per-element sums run in the same
  // order either way
  constexpr int NPG0 = NODES * 128 / NT;
  constexpr int NPG = NODES < 8 ? NODES : (NPG0 >= 8 ? 8 : (NPG0 < 1 ? 1 : NPG0));
  constexpr int NGRP = NODES / NPG;
  const int H = P.hidden;
  for (int item = threadIdx.x; item < NGRP * H; item += NT) {
    const int i = item % H;
    const int g0 = (item / H) * NPG;
    float acc[NPG];
#pragma unroll
    for (int q = 0; q < NPG; ++q) acc[q] = 0.f;
    const float4* wr = reinterpret_cast<const float4*>(P.W1 + static_cast<int64_t>(i) * 2 * D);
#pragma unroll 4
    for (int k4 = 0; k4 < (2 * D) / 4; ++k4) {
      const float4 wv = wr[k4];
#pragma unroll
      for (int q = 0; q < NPG; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(&sm.feat[g0 + q][4 * k4]);
        acc[q] += wv.x * f.x + wv.y * f.y + wv.z * f.z + wv.w * f.w;
      }
    }
    const float b = P.b1[i];
#pragma unroll
    for (int q = 0; q < NPG; ++q) {
      const float z = acc[q] + b;
      sm.hid[g0 + q][i] = z / (1.0f + __expf(-z));
    }
  }
  __syncthreads();

  // ---- phase 3: m = W2 hid
  for (int item = threadIdx.x; item < NGRP * D; item += NT) {
    const int j = item % D;
    const int g0 = (item / D) * NPG;
    float acc[NPG];
#pragma unroll
    for (int q = 0; q < NPG; ++q) acc[q] = 0.f;
    const float4* wr = reinterpret_cast<const float4*>(P.W2 + static_cast<int64_t>(j) * H);
    for (int k4 = 0; k4 < H / 4; ++k4) {
      const float4 wv = wr[k4];
#pragma unroll
      for (int q = 0; q < NPG; ++q) {
        const float4 h = *reinterpret_cast<const float4*>(&sm.hid[g0 + q][4 * k4]);
        acc[q] += wv.x * h.x + wv.y * h.y + wv.z * h.z + wv.w * h.w;
      }
    }
#pragma unroll
    for (int q = 0; q < NPG; ++q) sm.m[g0 + q][j] = acc[q];
  }
  __syncthreads();
  }

  if constexpr (STATS) {
    // sigma and ||mu||^2 of each node next to its m (hid is free once the
    // MLP is done), then per-dimension sums over the tile's nodes in node order
#pragma unroll
    for (int nw = 0; nw < NPW; ++nw) {
      const int n = wid * NPW + nw;
      if (n < NODES && lane == 0) {
        sm.hid[n][0] = n < n_valid ? sig_r[nw] : 0.f;
        sm.hid[n][1] = n < n_valid ? mu2_r[nw] : 0.f;
      }
    }
    __syncthreads();
    for (int j = threadIdx.x; j <= D; j += NT) {
      float acc = 0.f;
      for (int n = 0; n < n_valid && n < NODES; ++n)
        acc += j < D ? sm.hid[n][0] * sm.m[n][j] : sm.hid[n][1];
      stats[j] = acc;
    }
    return;
  }

  // ---- phase 4: K = mu + g (p - mu) + sigma m
#pragma unroll
  for (int nw = 0; nw < NPW; ++nw) {
    const int n = wid * NPW + nw;
    if (n >= NODES || n >= n_valid) continue;
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      const float kv = mu_r[nw][u] + P.g * (p_r[nw][u] - mu_r[nw][u]) +
                       sig_r[nw] * sm.m[n][i0 + u];
      Stor<DT>::store(ko + static_cast<int64_t>(n) * D + i0 + u, kv);
      sm.m[n][i0 + u] = Stor<DT>::round(kv);         // the stored value, for phase 5
                                                      // (over the m element just read)
    }
  }
  __syncthreads();

  // ---- phase 5: rotated keys from the stored (rounded) node keys, when the
  // tree keeps them (kro null: not kept)
  if (kro == nullptr) return;
  constexpr int H2 = D / 2;
  for (int item = threadIdx.x; item < NODES * H2; item += NT) {
    const int n = item / H2, jj = item % H2;
    if (n >= n_valid) continue;
    const int c = (c0 + n) % kC;
    const float* rp = rope + (c * H2 + jj) * 2;
    float xo, yo;
    rope_pair(sm.m[n][jj], sm.m[n][jj + H2], rp[0], rp[1], xo, yo);
    Stor<DT>::store(kro + static_cast<int64_t>(n) * D + jj, xo);
    Stor<DT>::store(kro + static_cast<int64_t>(n) * D + jj + H2, yo);
  }
}

}  // namespace recsa
