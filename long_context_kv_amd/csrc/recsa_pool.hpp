// Pooling of C=16 children into one tree node (picx.dev Tree Construction,
// Eq. 1 for values; Pooler Distillation, Eq. 5 for keys), for a tile of
// NODES consecutive nodes and a workgroup of NT threads.  Arithmetic is
// float32; the node is rounded once to the storage dtype when stored.
#pragma once

#include "recsa_common.hpp"

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
template <int DT, int D, int NODES>
struct PoolSmem {
  float feat[NODES][2 * D];
  float hid[NODES][256];
  float m[NODES][D];
};

template <int DT, int D, int NODES, int NT, bool STATS = false>
__device__ void pool_tile(const typename Stor<DT>::T* __restrict__ kc,  // child K rows
                          const typename Stor<DT>::T* __restrict__ vc,  // child V rows
                          typename Stor<DT>::T* __restrict__ ko,        // node K rows
                          typename Stor<DT>::T* __restrict__ vo,        // node V rows
                          typename Stor<DT>::T* __restrict__ kro,       // rotated node K rows
                          int c0,                   // index mod C of the tile's first node
                          const float* __restrict__ rope,
                          int n_valid, const recsa_pooler& P,
                          PoolSmem<DT, D, NODES>& sm, float* __restrict__ stats = nullptr) {
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
#pragma unroll
    for (int c = 0; c < kC; ++c) a[c] = wave_sum(a[c]);
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

  if constexpr (STATS) {
    // sigma and ||mu||^2 of each node next to its m (feat is free after
    // phase 2), then per-dimension sums over the tile's nodes in node order
#pragma unroll
    for (int nw = 0; nw < NPW; ++nw) {
      const int n = wid * NPW + nw;
      if (n < NODES && lane == 0) {
        sm.feat[n][0] = n < n_valid ? sig_r[nw] : 0.f;
        sm.feat[n][1] = n < n_valid ? mu2_r[nw] : 0.f;
      }
    }
    __syncthreads();
    for (int j = threadIdx.x; j <= D; j += NT) {
      float acc = 0.f;
      for (int n = 0; n < n_valid && n < NODES; ++n)
        acc += j < D ? sm.feat[n][0] * sm.m[n][j] : sm.feat[n][1];
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
      sm.feat[n][i0 + u] = Stor<DT>::round(kv);      // the stored value, for phase 5
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
    rope_pair(sm.feat[n][jj], sm.feat[n][jj + H2], rp[0], rp[1], xo, yo);
    Stor<DT>::store(kro + static_cast<int64_t>(n) * D + jj, xo);
    Stor<DT>::store(kro + static_cast<int64_t>(n) * D + jj + H2, yo);
  }
}

}  // namespace recsa
