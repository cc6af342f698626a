// Tree construction kernels: RoPE table, level pooling (build) and decode
// append.  Node value = mean of the C children values (picx.dev Tree
// Construction, Eq. 1); node key = pooler of the C children keys (Pooler
// Distillation, Eq. 5).  Arithmetic is float32; nodes are rounded once to the
// storage dtype when stored, and every level reads the stored children.
#include <algorithm>

#include "recsa_common.hpp"
#include "recsa_kernels.hpp"

namespace recsa {

// ------------------------------------------------------------ RoPE table
__global__ void __launch_bounds__(kBlock) rope_table_kernel(float* table, int d, int n_pos,
                                                            double theta) {
  const int half = d / 2;
  const int64_t n = static_cast<int64_t>(n_pos) * half;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kBlock) {
    const int phi = static_cast<int>(i / half);
    const int j = static_cast<int>(i % half);
    const double inv_freq = pow(theta, (-2.0 * j) / d);
    const double ang = static_cast<double>(phi) * inv_freq;
    table[2 * i] = static_cast<float>(cos(ang));
    table[2 * i + 1] = static_cast<float>(sin(ang));
  }
}

// ---------------------------------------------------------- pooling tile
// One workgroup pools NODES consecutive nodes of one (sequence, KV head).
// Phase 1 (one wave per node): children statistics, alpha, p, value mean.
// Phase 2/3 (all threads): the pooler MLP for the tile, weights streamed
// from L2 once per tile.  Phase 4: K = mu + g (p - mu) + sigma m.
template <int DT, int D, int NODES>
struct PoolSmem {
  float feat[NODES][2 * D];
  float hid[NODES][256];
  float m[NODES][D];
};

template <int DT, int D, int NODES>
__device__ void pool_tile(const typename Stor<DT>::T* __restrict__ kc,  // child K rows
                          const typename Stor<DT>::T* __restrict__ vc,  // child V rows
                          typename Stor<DT>::T* __restrict__ ko,        // node K rows
                          typename Stor<DT>::T* __restrict__ vo,        // node V rows
                          int n_valid, const recsa_pooler& P,
                          PoolSmem<DT, D, NODES>& sm) {
  using T = typename Stor<DT>::T;
  constexpr int DPL = D / kWave;                 // dims per lane (1 or 2)
  constexpr int NPW = (NODES + 3) / 4;           // nodes per wave
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x >> 6;
  const int i0 = lane * DPL;

  float mu_r[NPW][DPL], p_r[NPW][DPL], sig_r[NPW];

  // ---- phase 1
#pragma unroll
  for (int nw = 0; nw < NPW; ++nw) {
    const int n = wid * NPW + nw;
    sig_r[nw] = 0.f;
    if (n >= NODES || n >= n_valid) continue;
    float x[kC][DPL];
    float vs[DPL];
#pragma unroll
    for (int u = 0; u < DPL; ++u) vs[u] = 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const T* kr = kc + (static_cast<int64_t>(n) * kC + c) * D + i0;
      const T* vr = vc + (static_cast<int64_t>(n) * kC + c) * D + i0;
      float tmp[2];
      if constexpr (DPL == 2) {
        load_vec<DT, 2>(kr, x[c]);
        load_vec<DT, 2>(vr, tmp);
        vs[0] += tmp[0];
        vs[1] += tmp[1];
      } else {
        x[c][0] = Stor<DT>::load(kr);
        vs[0] += Stor<DT>::load(vr);
      }
    }
    // value mean (Eq. 1)
#pragma unroll
    for (int u = 0; u < DPL; ++u)
      Stor<DT>::store(vo + static_cast<int64_t>(n) * D + i0 + u, vs[u] * (1.0f / kC));
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
    for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
      for (int c = 0; c < kC; ++c) a[c] += __shfl_xor(a[c], o, kWave);
    }
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
  }
  __syncthreads();

  // ---- phase 2: hid = SiLU(W1 feat + b1)
  constexpr int NPG = NODES < 8 ? NODES : 8;     // nodes per thread
  constexpr int NGRP = NODES / NPG;
  const int H = P.hidden;
  for (int item = threadIdx.x; item < NGRP * H; item += kBlock) {
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
  for (int item = threadIdx.x; item < NGRP * D; item += kBlock) {
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
    }
  }
}

// Build nodes [n_lo, n_hi) of `level` for every (sequence, KV head).
template <int DT, int D>
__global__ void __launch_bounds__(kBlock) build_level_kernel(recsa_tree tr, recsa_pooler P,
                                                             int level, int64_t n_lo,
                                                             int64_t n_hi) {
  using T = typename Stor<DT>::T;
  constexpr int NODES = 16;
  __shared__ PoolSmem<DT, D, NODES> sm;
  const int j = blockIdx.y, b = blockIdx.z;
  const int64_t first = n_lo + static_cast<int64_t>(blockIdx.x) * NODES;
  const int n_valid = static_cast<int>(min<int64_t>(NODES, n_hi - first));
  const int64_t rows_up = level_rows_dev(tr.L_cap, level - 1);
  const int64_t rows = level_rows_dev(tr.L_cap, level);
  const int64_t head = static_cast<int64_t>(b) * tr.Hkv + j;
  const T* kc = static_cast<const T*>(tr.K[level - 1]) + (head * rows_up + first * kC) * D;
  const T* vc = static_cast<const T*>(tr.V[level - 1]) + (head * rows_up + first * kC) * D;
  T* ko = static_cast<T*>(tr.K[level]) + (head * rows + first) * D;
  T* vo = static_cast<T*>(tr.V[level]) + (head * rows + first) * D;
  pool_tile<DT, D, NODES>(kc, vc, ko, vo, n_valid, P, sm);
}

// Decode append: write row t, then complete each node whose last token is t.
template <int DT, int D>
__global__ void __launch_bounds__(kBlock) append_kernel(recsa_tree tr, recsa_pooler P,
                                                        const void* k_new, const void* v_new,
                                                        const int64_t* pos) {
  using T = typename Stor<DT>::T;
  __shared__ PoolSmem<DT, D, 1> sm;
  const int j = blockIdx.x, b = blockIdx.y;
  const int64_t head = static_cast<int64_t>(b) * tr.Hkv + j;
  const int64_t t = pos[b];
  {
    const T* ks = static_cast<const T*>(k_new) + head * D;
    const T* vs = static_cast<const T*>(v_new) + head * D;
    T* kd = static_cast<T*>(tr.K[0]) + (head * tr.L_cap + t) * D;
    T* vd = static_cast<T*>(tr.V[0]) + (head * tr.L_cap + t) * D;
    for (int i = threadIdx.x; i < D; i += kBlock) {
      kd[i] = ks[i];
      vd[i] = vs[i];
    }
  }
  int64_t span = 1;
  for (int l = 1; l < tr.n_levels; ++l) {
    span *= kC;
    if ((t + 1) % span != 0) break;
    __threadfence();
    __syncthreads();
    const int64_t node = (t + 1) / span - 1;
    const int64_t rows_up = level_rows_dev(tr.L_cap, l - 1);
    const int64_t rows = level_rows_dev(tr.L_cap, l);
    const T* kc = static_cast<const T*>(tr.K[l - 1]) + (head * rows_up + node * kC) * D;
    const T* vc = static_cast<const T*>(tr.V[l - 1]) + (head * rows_up + node * kC) * D;
    T* ko = static_cast<T*>(tr.K[l]) + (head * rows + node) * D;
    T* vo = static_cast<T*>(tr.V[l]) + (head * rows + node) * D;
    pool_tile<DT, D, 1>(kc, vc, ko, vo, 1, P, sm);
    __syncthreads();
  }
}

// ------------------------------------------------------------- launchers
hipError_t launch_rope_table(float* table, int d, int n_pos, double theta, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(n_pos) * (d / 2);
  const int grid = static_cast<int>(std::min<int64_t>((n + kBlock - 1) / kBlock, 4096));
  rope_table_kernel<<<grid, kBlock, 0, s>>>(table, d, n_pos, theta);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t build_impl(const recsa_tree& tr, const recsa_pooler& P, int64_t tb, int64_t te,
                             hipStream_t s) {
  int64_t span = 1;
  for (int l = 1; l < tr.n_levels; ++l) {
    span *= kC;
    const int64_t rows = level_rows_host(tr.L_cap, l);
    const int64_t n_lo = tb / span;
    const int64_t n_hi = std::min<int64_t>(te / span, rows);
    if (n_hi <= n_lo) continue;
    const int64_t tiles = (n_hi - n_lo + 15) / 16;
    dim3 grid(static_cast<unsigned>(tiles), tr.Hkv, tr.B);
    build_level_kernel<DT, D><<<grid, kBlock, 0, s>>>(tr, P, l, n_lo, n_hi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_build(const recsa_tree& tr, const recsa_pooler& P, int64_t tb, int64_t te,
                        hipStream_t s) {
  if (tr.dtype == RECSA_BF16)
    return tr.d == 128 ? build_impl<RECSA_BF16, 128>(tr, P, tb, te, s)
                       : build_impl<RECSA_BF16, 64>(tr, P, tb, te, s);
  return tr.d == 128 ? build_impl<RECSA_F32, 128>(tr, P, tb, te, s)
                     : build_impl<RECSA_F32, 64>(tr, P, tb, te, s);
}

hipError_t launch_append(const recsa_tree& tr, const recsa_pooler& P, const void* k_new,
                         const void* v_new, const int64_t* pos, hipStream_t s) {
  dim3 grid(tr.Hkv, tr.B);
  if (tr.dtype == RECSA_BF16) {
    if (tr.d == 128)
      append_kernel<RECSA_BF16, 128><<<grid, kBlock, 0, s>>>(tr, P, k_new, v_new, pos);
    else
      append_kernel<RECSA_BF16, 64><<<grid, kBlock, 0, s>>>(tr, P, k_new, v_new, pos);
  } else {
    if (tr.d == 128)
      append_kernel<RECSA_F32, 128><<<grid, kBlock, 0, s>>>(tr, P, k_new, v_new, pos);
    else
      append_kernel<RECSA_F32, 64><<<grid, kBlock, 0, s>>>(tr, P, k_new, v_new, pos);
  }
  return hipGetLastError();
}

}  // namespace recsa
