// Pooler backward: gradients of the pooler parameters (picx.dev Pooler
// Distillation, Eq. 5; trained with Eq. 6 and Eq. 7, Training Stages stage 1)
// for the complete nodes of one level, given an upstream gradient of each
// node key and, optionally, the level's shift penalty (Eq. 7) with a weight.
//
// L = sum_i dK_i . K_i + lambda * penalty, with
//   K = mu + g (p - mu) + sigma m,  m = W2 SiLU(z),  z = W1 [mu/rho ; (p-mu)/sigma] + b1,
//   p = sum_c alpha_c x_c,  alpha = softmax_c(tau u_c),  u_c = w.(x_c - mu)/sigma.
// The children x are inputs (each level is pooled from stored rows), so mu,
// sigma and rho carry no gradient; rounding the stored key is taken as the
// identity.  The penalty reaches the parameters only through m:
//   d penalty / d m_i = 2 sigma_i S / (M U),  S = sum sigma m,  U = sum ||mu||^2.
//
// pool_bwd_tile_kernel: one workgroup per 16 nodes of one (sequence, KV
//   head) recomputes the forward parts and writes, per node, the rows the
//   weight gradients contract over (feat, dm, dz, SiLU(z)), and per tile the
//   sums of the w, tau and g gradients.
// pool_bwd_chunk_kernel + pool_bwd_reduce_kernel: each output element sums
//   its node rows (or tile partials) in chunks of 512 rows, then the chunks,
//   in float64 and in a fixed order: identical bits on every call.
#include <algorithm>

#include "recsa_common.hpp"
#include "recsa_kernels.hpp"

namespace recsa {

namespace {

constexpr int kBwdNodes = 16;

template <int D>
struct PoolBwdSmem {
  alignas(16) float feat[kBwdNodes][2 * D];   // read as float4
  float z[kBwdNodes][256];
  float dz[kBwdNodes][256];
  float dm[kBwdNodes][D];
  float dk[kBwdNodes][D];      // dK, then dp
  float pmu[kBwdNodes][D];     // p - mu, then the node's w gradient
  float alpha[kBwdNodes][kC];
  float u[kBwdNodes][kC];
  float sig[kBwdNodes];
  float dtau[kBwdNodes];
  float red[kBlock / kWave];
};

__device__ __forceinline__ float bwd_block_sum(float v, float* red) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kBlock / kWave; ++w) s += red[w];
  return s;
}

}  // namespace

// Row of one node in the workspace: feat [2D], dm [D], dz [H], SiLU(z) [H].
__host__ __device__ inline int64_t bwd_row_floats(int D, int H) { return 3 * D + 2 * H; }

template <int DT, int D>
__global__ void __launch_bounds__(kBlock) pool_bwd_tile_kernel(
    recsa_tree tr, recsa_pooler P, int level, int64_t n_nodes, const float* __restrict__ dK,
    const float* __restrict__ shift_sums, float shift_coef, float* __restrict__ rows,
    float* __restrict__ part) {
  using Ty = typename Stor<DT>::T;
  constexpr int DPL = D / kWave;
  constexpr int NW = kBlock / kWave;
  constexpr int NPW = kBwdNodes / NW;
  __shared__ PoolBwdSmem<D> sm;
  const int H = P.hidden;
  const int j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid >> 6;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kBwdNodes;
  const int n_valid = static_cast<int>(min<int64_t>(kBwdNodes, n_nodes - first));
  const int64_t head = static_cast<int64_t>(b) * tr.Hkv + j;
  const int64_t rows_up = level_rows_dev(tr.L_cap, level - 1);
  const int64_t rows_l = level_rows_dev(tr.L_cap, level);
  const Ty* kc = static_cast<const Ty*>(tr.K[level - 1]) + (head * rows_up + first * kC) * D;
  const int i0 = lane * DPL;
  // 2 lambda / (M U): the penalty's gradient per unit of sigma_i S
  const float cu = shift_sums ? shift_coef / shift_sums[D] : 0.f;

  // ---- F1: children statistics, one wave per node
  float mu_r[NPW][DPL];
#pragma unroll
  for (int nw = 0; nw < NPW; ++nw) {
    const int n = wid * NPW + nw;
#pragma unroll
    for (int v = 0; v < DPL; ++v) mu_r[nw][v] = 0.f;
    if (n >= n_valid) {
#pragma unroll
      for (int v = 0; v < DPL; ++v) {
        sm.feat[n][i0 + v] = 0.f;
        sm.feat[n][D + i0 + v] = 0.f;
        sm.dk[n][i0 + v] = 0.f;
        sm.pmu[n][i0 + v] = 0.f;
      }
      if (lane < kC) {
        sm.alpha[n][lane] = 0.f;
        sm.u[n][lane] = 0.f;
      }
      if (lane == 0) sm.sig[n] = 0.f;
      continue;
    }
    float x[kC][DPL];
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const Ty* xr = kc + (static_cast<int64_t>(n) * kC + c) * D + i0;
      if constexpr (DPL == 2)
        load_vec<DT, 2>(xr, x[c]);
      else
        x[c][0] = Stor<DT>::load(xr);
    }
    float mu[DPL];
#pragma unroll
    for (int v = 0; v < DPL; ++v) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kC; ++c) s += x[c][v];
      mu[v] = s * (1.0f / kC);
      mu_r[nw][v] = mu[v];
    }
    float sq = 0.f, mq = 0.f;
#pragma unroll
    for (int v = 0; v < DPL; ++v) {
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        const float dv = x[c][v] - mu[v];
        sq += dv * dv;
      }
      mq += mu[v] * mu[v];
    }
    sq = wave_sum(sq);
    mq = wave_sum(mq);
    const float sigma = sqrtf(sq / static_cast<float>(kC * D) + P.eps);
    const float rho = sqrtf(mq / static_cast<float>(D) + P.eps);
    const float inv_sig = 1.0f / sigma;
    float a[kC];
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < DPL; ++v) s += P.w[i0 + v] * (x[c][v] - mu[v]);
      a[c] = wave_sum(s) * inv_sig;          // u_c
    }
    float amax = -INFINITY;
#pragma unroll
    for (int c = 0; c < kC; ++c) amax = fmaxf(amax, P.tau * a[c]);
    float e[kC], esum = 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      e[c] = expf(P.tau * a[c] - amax);
      esum += e[c];
    }
    const float inv = 1.0f / esum;
    float p[DPL];
#pragma unroll
    for (int v = 0; v < DPL; ++v) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kC; ++c) s += e[c] * x[c][v];
      p[v] = s * inv;
    }
    const float* dkr = dK ? dK + (head * rows_l + first + n) * D : nullptr;
#pragma unroll
    for (int v = 0; v < DPL; ++v) {
      sm.feat[n][i0 + v] = mu[v] / rho;
      sm.feat[n][D + i0 + v] = (p[v] - mu[v]) * inv_sig;
      sm.pmu[n][i0 + v] = p[v] - mu[v];
      sm.dk[n][i0 + v] = dkr ? dkr[i0 + v] : 0.f;
    }
    // every lane holds all C values; lane c publishes its own
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      if (lane == c) {
        sm.alpha[n][c] = e[c] * inv;
        sm.u[n][c] = a[c];
      }
    }
    if (lane == 0) sm.sig[n] = sigma;
  }
  __syncthreads();

  // ---- F2: z = W1 feat + b1
  for (int item = tid; item < 2 * H; item += kBlock) {
    const int i = item % H, g0 = (item / H) * 8;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    const float4* wr = reinterpret_cast<const float4*>(P.W1 + static_cast<int64_t>(i) * 2 * D);
    for (int k4 = 0; k4 < (2 * D) / 4; ++k4) {
      const float4 wv = wr[k4];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(&sm.feat[g0 + q][4 * k4]);
        acc[q] += wv.x * f.x + wv.y * f.y + wv.z * f.z + wv.w * f.w;
      }
    }
    const float bias = P.b1[i];
#pragma unroll
    for (int q = 0; q < 8; ++q) sm.z[g0 + q][i] = acc[q] + bias;
  }
  // ---- B1: dm = sigma dK + (shift) coef sigma S;  g gradient of the tile
  float gpart = 0.f;
  for (int item = tid; item < kBwdNodes * D; item += kBlock) {
    const int n = item / D, jj = item % D;
    const float sv = shift_sums ? shift_sums[jj] : 0.f;
    sm.dm[n][jj] = sm.sig[n] * sm.dk[n][jj] + cu * sm.sig[n] * sv;
    gpart += sm.dk[n][jj] * sm.pmu[n][jj];
  }
  const float g_tile = bwd_block_sum(gpart, sm.red);   // includes the barrier F2/B1 need

  // ---- B2: dz = (W2^T dm) SiLU'(z); node rows out
  for (int item = tid; item < 2 * H; item += kBlock) {
    const int i = item % H, g0 = (item / H) * 8;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    for (int jj = 0; jj < D; ++jj) {
      const float wv = P.W2[static_cast<int64_t>(jj) * H + i];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += wv * sm.dm[g0 + q][jj];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float zz = sm.z[g0 + q][i];
      const float s = 1.0f / (1.0f + expf(-zz));
      sm.dz[g0 + q][i] = acc[q] * (s * (1.0f + zz * (1.0f - s)));
      sm.z[g0 + q][i] = zz * s;                       // SiLU(z), for the W2 gradient
    }
  }
  __syncthreads();
  const int64_t RF = bwd_row_floats(D, H);
  float* rbase = rows + ((head * gridDim.x + blockIdx.x) * kBwdNodes) * RF;
  for (int n = 0; n < kBwdNodes; ++n) {
    float* r = rbase + n * RF;
    for (int e = tid; e < 2 * D; e += kBlock) r[e] = sm.feat[n][e];
    for (int e = tid; e < D; e += kBlock) r[2 * D + e] = sm.dm[n][e];
    for (int e = tid; e < H; e += kBlock) {
      r[3 * D + e] = sm.dz[n][e];
      r[3 * D + H + e] = sm.z[n][e];
    }
  }
  // ---- B3: dp = g dK + (W1[:, D:]^T dz) / sigma   (into dk)
  for (int item = tid; item < 2 * D; item += kBlock) {
    const int jj = item % D, g0 = (item / D) * 8;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    for (int i = 0; i < H; ++i) {
      const float wv = P.W1[static_cast<int64_t>(i) * 2 * D + D + jj];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += wv * sm.dz[g0 + q][i];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int n = g0 + q;
      const float s = sm.sig[n];
      sm.dk[n][jj] = P.g * sm.dk[n][jj] + (s > 0.f ? acc[q] / s : 0.f);
    }
  }
  __syncthreads();

  // ---- B4: through alpha to tau and w, one wave per node
#pragma unroll
  for (int nw = 0; nw < NPW; ++nw) {
    const int n = wid * NPW + nw;
    if (n >= n_valid) {
#pragma unroll
      for (int v = 0; v < DPL; ++v) sm.pmu[n][i0 + v] = 0.f;
      if (lane == 0) sm.dtau[n] = 0.f;
      continue;
    }
    float x[kC][DPL];
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const Ty* xr = kc + (static_cast<int64_t>(n) * kC + c) * D + i0;
      if constexpr (DPL == 2)
        load_vec<DT, 2>(xr, x[c]);
      else
        x[c][0] = Stor<DT>::load(xr);
    }
    float da[kC], asum = 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < DPL; ++v) s += sm.dk[n][i0 + v] * x[c][v];
      da[c] = wave_sum(s);                           // d alpha_c
      asum += sm.alpha[n][c] * da[c];
    }
    float tpart = 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      da[c] = sm.alpha[n][c] * (da[c] - asum);       // d (tau u_c)
      tpart += da[c] * sm.u[n][c];
    }
    const float inv_sig = 1.0f / sm.sig[n];
#pragma unroll
    for (int v = 0; v < DPL; ++v) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kC; ++c) s += da[c] * (x[c][v] - mu_r[nw][v]);
      sm.pmu[n][i0 + v] = P.tau * s * inv_sig;       // this node's w gradient
    }
    if (lane == 0) sm.dtau[n] = tpart;
  }
  __syncthreads();
  float* pp = part + (head * gridDim.x + blockIdx.x) * (D + 2);
  for (int jj = tid; jj < D; jj += kBlock) {
    float s = 0.f;
    for (int n = 0; n < kBwdNodes; ++n) s += sm.pmu[n][jj];
    pp[jj] = s;
  }
  if (tid == 0) {
    float s = 0.f;
    for (int n = 0; n < kBwdNodes; ++n) s += sm.dtau[n];
    pp[D] = s;
    pp[D + 1] = g_tile;
  }
}

// Output element e of [dW1 (H x 2D) | dW2 (D x H) | db1 (H) | dw (D) | dtau | dg].
// Stage 1: workgroup (x, c) sums node rows [c*kBwdChunk, (c+1)*kBwdChunk)
// (and their tiles' partials) for 256 output elements, in float64, into
// acc[c][e].  Stage 2: each element sums its chunks in order.  Both orders
// are fixed: identical bits on every call.
constexpr int kBwdChunk = 512;            // node rows per stage-1 workgroup (32 tiles)

__host__ __device__ inline int64_t bwd_outputs(int D, int H) {
  return static_cast<int64_t>(H) * 3 * D + H + D + 2;
}

template <int D>
__global__ void __launch_bounds__(kBlock) pool_bwd_chunk_kernel(
    const float* __restrict__ rows, const float* __restrict__ part, int64_t n_rows, int H,
    double* __restrict__ acc_out) {
  const int64_t RF = bwd_row_floats(D, H);
  const int64_t n_w1 = static_cast<int64_t>(H) * 2 * D, n_w2 = static_cast<int64_t>(D) * H;
  const int64_t total = bwd_outputs(D, H);
  const int64_t e = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kBwdChunk;
  const int64_t r1 = min(r0 + kBwdChunk, n_rows);
  if (e >= total) return;
  double acc = 0.0;
  if (e < n_w1) {                                   // dW1[i][k] = sum dz_i feat_k
    const int i = static_cast<int>(e / (2 * D)), k = static_cast<int>(e % (2 * D));
    for (int64_t r = r0; r < r1; ++r)
      acc += static_cast<double>(rows[r * RF + 3 * D + i]) * rows[r * RF + k];
  } else if (e < n_w1 + n_w2) {                     // dW2[jj][i] = sum dm_jj SiLU(z)_i
    const int64_t f = e - n_w1;
    const int jj = static_cast<int>(f / H), i = static_cast<int>(f % H);
    for (int64_t r = r0; r < r1; ++r)
      acc += static_cast<double>(rows[r * RF + 2 * D + jj]) * rows[r * RF + 3 * D + H + i];
  } else if (e < n_w1 + n_w2 + H) {                 // db1[i] = sum dz_i
    const int i = static_cast<int>(e - n_w1 - n_w2);
    for (int64_t r = r0; r < r1; ++r) acc += rows[r * RF + 3 * D + i];
  } else {                                          // dw, dtau, dg from the tile sums
    const int c = static_cast<int>(e - n_w1 - n_w2 - H);
    for (int64_t t = r0 / kBwdNodes; t < r1 / kBwdNodes; ++t) acc += part[t * (D + 2) + c];
  }
  acc_out[static_cast<int64_t>(blockIdx.y) * total + e] = acc;
}

template <int D>
__global__ void __launch_bounds__(kBlock) pool_bwd_reduce_kernel(const double* __restrict__ acc_in,
                                                                 int n_chunks, int H,
                                                                 recsa_pooler_grad G) {
  const int64_t n_w1 = static_cast<int64_t>(H) * 2 * D, n_w2 = static_cast<int64_t>(D) * H;
  const int64_t total = bwd_outputs(D, H);
  const int64_t e = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x;
  if (e >= total) return;
  double acc = 0.0;
  for (int c = 0; c < n_chunks; ++c) acc += acc_in[static_cast<int64_t>(c) * total + e];
  const float v = static_cast<float>(acc);
  if (e < n_w1) {
    G.W1[e] = v;
  } else if (e < n_w1 + n_w2) {
    G.W2[e - n_w1] = v;
  } else if (e < n_w1 + n_w2 + H) {
    G.b1[e - n_w1 - n_w2] = v;
  } else {
    const int c = static_cast<int>(e - n_w1 - n_w2 - H);
    if (c < D)
      G.w[c] = v;
    else if (c == D)
      G.tau[0] = v;
    else
      G.g[0] = v;
  }
}

// ------------------------------------------------------------ launchers
struct BwdLayout {
  int64_t tiles, n_rows, n_parts, n_chunks, rows_off, part_off, acc_off, total;
};

static BwdLayout bwd_layout(const recsa_tree& tr, int H, int level, int64_t n_nodes) {
  BwdLayout L;
  const int64_t heads = static_cast<int64_t>(tr.B) * tr.Hkv;
  L.tiles = (n_nodes + kBwdNodes - 1) / kBwdNodes;
  L.n_rows = L.tiles * kBwdNodes * heads;
  L.n_parts = L.tiles * heads;
  L.n_chunks = (L.n_rows + kBwdChunk - 1) / kBwdChunk;
  L.rows_off = 0;
  L.part_off = align256(L.n_rows * bwd_row_floats(tr.d, H) * 4);
  L.acc_off = align256(L.part_off + L.n_parts * (tr.d + 2) * 4);
  L.total = L.acc_off + std::max<int64_t>(L.n_chunks, 1) * bwd_outputs(tr.d, H) * 8;
  (void)level;
  return L;
}

int64_t pool_bwd_ws_bytes(const recsa_tree& tr, const recsa_pooler& P, int level) {
  return bwd_layout(tr, P.hidden, level, level_rows_host(tr.L_cap, level)).total;
}

template <int DT, int D>
static hipError_t pool_bwd_impl(const recsa_tree& tr, const recsa_pooler& P, int level,
                                int64_t tok_end, const float* dK, const float* shift_sums,
                                float shift_weight, const recsa_pooler_grad& G, void* ws,
                                hipStream_t s) {
  const int64_t n = std::min(tok_end >> (4 * level), level_rows_host(tr.L_cap, level));
  const BwdLayout L = bwd_layout(tr, P.hidden, level, n);
  float* rows = reinterpret_cast<float*>(static_cast<char*>(ws) + L.rows_off);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + L.part_off);
  const int64_t M = n * tr.B * tr.Hkv;
  // d penalty / d m_i = sigma_i * (2 lambda / (M U)) * S; U read on the device
  const float coef = M > 0 ? 2.0f * shift_weight / static_cast<float>(M) : 0.f;
  if (n > 0) {
    dim3 grid(static_cast<unsigned>(L.tiles), tr.Hkv, tr.B);
    pool_bwd_tile_kernel<DT, D><<<grid, kBlock, 0, s>>>(tr, P, level, n, dK, shift_sums, coef,
                                                        rows, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  double* acc = reinterpret_cast<double*>(static_cast<char*>(ws) + L.acc_off);
  const int64_t total = bwd_outputs(D, P.hidden);
  const unsigned gx = static_cast<unsigned>((total + kBlock - 1) / kBlock);
  const int n_chunks = n > 0 ? static_cast<int>(L.n_chunks) : 1;
  pool_bwd_chunk_kernel<D><<<dim3(gx, n_chunks), kBlock, 0, s>>>(rows, part, n > 0 ? L.n_rows : 0,
                                                                 P.hidden, acc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  pool_bwd_reduce_kernel<D><<<gx, kBlock, 0, s>>>(acc, n_chunks, P.hidden, G);
  return hipGetLastError();
}

hipError_t launch_pool_backward(const recsa_tree& tr, const recsa_pooler& P, int level,
                                int64_t tok_end, const float* dK, const float* shift_sums,
                                float shift_weight, const recsa_pooler_grad& G, void* ws,
                                hipStream_t s) {
  if (tr.dtype == RECSA_BF16)
    return tr.d == 128 ? pool_bwd_impl<RECSA_BF16, 128>(tr, P, level, tok_end, dK, shift_sums,
                                                        shift_weight, G, ws, s)
                       : pool_bwd_impl<RECSA_BF16, 64>(tr, P, level, tok_end, dK, shift_sums,
                                                       shift_weight, G, ws, s);
  return tr.d == 128 ? pool_bwd_impl<RECSA_F32, 128>(tr, P, level, tok_end, dK, shift_sums,
                                                     shift_weight, G, ws, s)
                     : pool_bwd_impl<RECSA_F32, 64>(tr, P, level, tok_end, dK, shift_sums,
                                                    shift_weight, G, ws, s);
}

}  // namespace recsa
