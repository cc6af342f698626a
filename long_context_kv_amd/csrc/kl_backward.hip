// Gradient of the Eq. 6 terms with respect to the node keys (picx.dev Pooler
// Distillation, Eq. 6: the student importance pi is trained toward the
// teacher's subtree mass y; the keys come from the pooler of Eq. 5, so this
// is the key gradient recsa_pooler_backward takes as dK).
//
// With P_h = softmax_h(s_h) over a level's non-current candidates, pi =
// mean_h P_h and r = y / pi:
//   d KL / d s_h,e = -(P_h,e / G) (r_e - sum_f r_f P_h,f),
// and s_h,e = q~_h . k~_e / sqrt(d) with the split candidate-local RoPE gives
//   d s_h,e / d K_e = R(c_e)^T q~_h / sqrt(d)
// (the operand roundings taken as the identity; q~_h = rnd(R(phi) q_h) exactly
// as the forward scoring forms it).  Each key collects these terms over every
// (query, head) whose list holds it as a non-current candidate.
//
// kgrad_coef_kernel   per (query, KV head, scored level): the coefficients
//                     d KL / d s_h,e from the selection logits, pi and y.
// kgrad_accum_kernel  per (sequence, KV head, level, parent node w, chunk of
//                     2048 queries): walks the chunk's queries in order, finds
//                     w among each query's parents, and accumulates coefficient
//                     x rotated query for w's 16 children.
// kgrad_finish_kernel per parent: the chunks in order, R(c)^T / sqrt(d), the
//                     rows out.  Fixed orders: identical bits on every call.
#include <math.h>

#include <algorithm>

#include "recsa_common.hpp"
#include "recsa_kernels.hpp"

namespace recsa {

namespace {

constexpr int kKgMatch = 8;        // matched queries per accumulation step
constexpr int kKgChunk = 2048;     // queries per accumulation workgroup

__device__ __forceinline__ float kg_block_max(float v, float* red) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kBlock / kWave; ++w) m = fmaxf(m, red[w]);
  return m;
}
__device__ __forceinline__ float kg_block_sum(float v, float* red) {
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

// coef: [n_queries * Hkv][n_sel][G][C*k], like the selection logits.
template <int G>
__global__ void __launch_bounds__(kBlock) kgrad_coef_kernel(
    recsa_tree tr, int T, const int64_t* __restrict__ pos, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, const float* __restrict__ imp,
    const float* __restrict__ teacher, const float* __restrict__ logits,
    float* __restrict__ coef) {
  __shared__ float red[kBlock / kWave];
  const int64_t qi = blockIdx.x;
  const int j = blockIdx.y, tid = threadIdx.x;
  const int n_sel = tr.n_levels - 1, k = tr.k, CK = kC * k, top = tr.n_levels - 1;
  const int64_t slot = qi * tr.Hkv + j;
  const int64_t t = pos[qi];
  const int32_t* sl = sel + slot * n_sel * k;
  const int32_t* cl = cnt + slot * n_sel;
  for (int l = 1; l <= n_sel; ++l) {
    const ListView lv = list_view(t, l, top, k, sl, cl);
    if (lv.len <= k) continue;                       // unscored (uniform)
    const int n = lv.len - 1;
    const int64_t base = (slot * n_sel + (l - 1)) * static_cast<int64_t>(CK);
    const float* yv = teacher + base;
    const float* pv = imp + base;
#pragma unroll 1
    for (int h = 0; h < G; ++h) {
      const float* s = logits + (slot * n_sel + (l - 1)) * static_cast<int64_t>(G) * CK +
                       static_cast<int64_t>(h) * CK;
      float m = -INFINITY;
      for (int p = tid; p < n; p += kBlock) m = fmaxf(m, s[p]);
      m = kg_block_max(m, red);
      float z = 0.f;
      for (int p = tid; p < n; p += kBlock) z += expf(s[p] - m);
      z = kg_block_sum(z, red);
      const float inv = 1.0f / z;
      float sr = 0.f;                                // sum_f r_f P_h,f
      for (int p = tid; p < n; p += kBlock) {
        const float r = pv[p] > 0.f ? yv[p] / pv[p] : 0.f;
        sr += r * (expf(s[p] - m) * inv);
      }
      sr = kg_block_sum(sr, red);
      float* cf = coef + (slot * n_sel + (l - 1)) * static_cast<int64_t>(G) * CK +
                  static_cast<int64_t>(h) * CK;
      for (int p = tid; p < n; p += kBlock) {
        const float r = pv[p] > 0.f ? yv[p] / pv[p] : 0.f;
        const float P = expf(s[p] - m) * inv;
        cf[p] = -(P / G) * (r - sr);
      }
    }
  }
}

// One workgroup per (parent node w of level l, chunk of kKgChunk queries) of
// one (sequence, KV head): the sum over the chunk's queries, in order, for
// w's children 16w .. 16w+15, before R(c)^T, into part[head][w][chunk][16][D].
// Thread (child c = tid / 16, dims DPT*(tid % 16) ...) owns DPT accumulators.
template <int DT, int D, int G>
__global__ void __launch_bounds__(kBlock) kgrad_accum_kernel(
    recsa_tree tr, const void* qv, int Hq, int T, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
    const float* __restrict__ coef, int level, int n_chunks, float* __restrict__ part) {
  using Ty = typename Stor<DT>::T;
  constexpr int H2 = D / 2;
  constexpr int DPT = D / 16;
  __shared__ float qt[kKgMatch][G][D];
  __shared__ float cf[kKgMatch][G][kC];
  __shared__ int m_qi[kBlock], m_rho[kBlock], m_nv[kBlock], m_phi[kBlock];
  __shared__ int red_i[kBlock / kWave];
  const int64_t w = blockIdx.x / n_chunks;
  const int chunk = static_cast<int>(blockIdx.x % n_chunks);
  const int j = blockIdx.y, b = blockIdx.z;
  const int64_t q_lo = static_cast<int64_t>(b) * T + static_cast<int64_t>(chunk) * kKgChunk;
  const int64_t q_hi = min(q_lo + kKgChunk, static_cast<int64_t>(b + 1) * T);
  const int tid = threadIdx.x;
  const int n_sel = tr.n_levels - 1, k = tr.k, CK = kC * k, top = tr.n_levels - 1;
  const int c_own = tid / 16, d0 = DPT * (tid % 16);
  float acc[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) acc[e] = 0.f;

  for (int64_t q0 = q_lo; q0 < q_hi; q0 += kBlock) {
    // ---- which queries of this batch hold w among their level-l parents
    const int64_t qi = q0 + tid;
    int rho = -1, nv = 0, phi = 0;
    if (qi < q_hi) {
      const int64_t slot = qi * tr.Hkv + j;
      const int64_t t = pos[qi];
      const ListView lv = list_view(t, level, top, k, sel + slot * n_sel * k, cnt + slot * n_sel);
      if (lv.len > k) {
        const int n = lv.len - 1;                    // non-current candidates
        if (lv.up) {
          const int ng = cnt[slot * n_sel + level];  // |S^(l+1)|
          int lo = 0, hi = ng - 1;
          while (lo <= hi) {
            const int mid = (lo + hi) >> 1;
            const int32_t v = lv.up[mid];
            if (v == w) {
              rho = mid;
              break;
            }
            if (v < w)
              lo = mid + 1;
            else
              hi = mid - 1;
          }
        } else if (kC * w < lv.len) {
          rho = static_cast<int>(w);
        }
        if (rho >= 0) {
          nv = min(kC, n - kC * rho);
          phi = (lv.len - 1) - kC * rho;
          if (nv <= 0) rho = -1;
        }
      }
    }
    int total;
    const int at = block_excl_scan(rho >= 0 ? 1 : 0, red_i, &total);
    if (rho >= 0) {
      m_qi[at] = static_cast<int>(qi - q0);
      m_rho[at] = rho;
      m_nv[at] = nv;
      m_phi[at] = phi;
    }
    __syncthreads();
    // ---- matched queries in order, kKgMatch at a time
    for (int m0 = 0; m0 < total; m0 += kKgMatch) {
      const int mc = min(kKgMatch, total - m0);
      // rotated, rounded query rows q~ = rnd(R(phi) q_h)
      for (int item = tid; item < kKgMatch * G * H2; item += kBlock) {
        const int m = item / (G * H2), h = (item / H2) % G, jj = item % H2;
        float xo = 0.f, yo = 0.f;
        if (m < mc) {
          const int64_t qq = q0 + m_qi[m0 + m];
          const Ty* qr = static_cast<const Ty*>(qv) + (qq * Hq + static_cast<int64_t>(j) * G + h) * D;
          const float* rp = tr.rope + (static_cast<int64_t>(m_phi[m0 + m]) * H2 + jj) * 2;
          rope_pair(Stor<DT>::load(qr + jj), Stor<DT>::load(qr + jj + H2), rp[0], rp[1], xo, yo);
          xo = Stor<DT>::round(xo);
          yo = Stor<DT>::round(yo);
        }
        qt[m][h][jj] = xo;
        qt[m][h][jj + H2] = yo;
      }
      for (int item = tid; item < kKgMatch * G * kC; item += kBlock) {
        const int m = item / (G * kC), h = (item / kC) % G, c = item % kC;
        float v = 0.f;
        if (m < mc && c < m_nv[m0 + m]) {
          const int64_t slot = (q0 + m_qi[m0 + m]) * tr.Hkv + j;
          v = coef[((slot * n_sel + (level - 1)) * G + h) * static_cast<int64_t>(CK) +
                   kC * m_rho[m0 + m] + c];
        }
        cf[m][h][c] = v;
      }
      __syncthreads();
      for (int m = 0; m < mc; ++m) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float a = cf[m][h][c_own];
#pragma unroll
          for (int e = 0; e < DPT; ++e) acc[e] += a * qt[m][h][d0 + e];
        }
      }
      __syncthreads();
    }
  }
  const int64_t n_par = gridDim.x / n_chunks;
  float* pp = part + (((static_cast<int64_t>(b) * tr.Hkv + j) * n_par + w) * n_chunks + chunk) *
                         (kC * D);
#pragma unroll
  for (int e = 0; e < DPT; ++e) pp[c_own * D + d0 + e] = acc[e];
}

// Per parent node: the chunks' sums in chunk order, then R(c)^T / sqrt(d) and
// the child rows out (every child row below rows_l, zero when no query scores
// it).
template <int D>
__global__ void __launch_bounds__(kBlock) kgrad_finish_kernel(recsa_tree tr, int level,
                                                              int n_chunks,
                                                              const float* __restrict__ part,
                                                              float* __restrict__ dK) {
  constexpr int H2 = D / 2;
  const int64_t w = blockIdx.x, n_par = gridDim.x;
  const int j = blockIdx.y, b = blockIdx.z;
  const int64_t rows_l = level_rows_dev(tr.L_cap, level);
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float* pp = part + ((static_cast<int64_t>(b) * tr.Hkv + j) * n_par + w) * n_chunks *
                               (kC * D);
  float* out = dK + (static_cast<int64_t>(b) * tr.Hkv + j) * rows_l * D;
  for (int item = threadIdx.x; item < kC * H2; item += kBlock) {
    const int c = item / H2, jj = item % H2;
    const int64_t u = kC * w + c;
    if (u >= rows_l) continue;
    float x = 0.f, y = 0.f;
    for (int ch = 0; ch < n_chunks; ++ch) {
      x += pp[static_cast<int64_t>(ch) * kC * D + c * D + jj];
      y += pp[static_cast<int64_t>(ch) * kC * D + c * D + jj + H2];
    }
    const float* rp = tr.rope + (static_cast<int64_t>(c) * H2 + jj) * 2;
    out[u * D + jj] = (x * rp[0] + y * rp[1]) * scale;
    out[u * D + jj + H2] = (-x * rp[1] + y * rp[0]) * scale;
  }
}

// ------------------------------------------------------------ launchers
// Workspace: the coefficients [n_queries*Hkv][n_sel][G][C*k], then the
// chunk sums of the largest level, [B*Hkv][parents][chunks][16][d].
static int64_t kgrad_coef_bytes(const recsa_tree& tr, int Hq, int64_t n_queries) {
  const int n_sel = tr.n_levels > 1 ? tr.n_levels - 1 : 1;
  return align256(n_queries * tr.Hkv * n_sel * static_cast<int64_t>(Hq / tr.Hkv) * kC * tr.k * 4);
}

static int64_t kgrad_chunks(const recsa_tree& tr, int64_t n_queries) {
  const int64_t T = n_queries / tr.B;
  return (T + kKgChunk - 1) / kKgChunk;
}

int64_t kgrad_ws_bytes(const recsa_tree& tr, int Hq, int64_t n_queries) {
  const int64_t parents = (level_rows_host(tr.L_cap, 1) + kC - 1) / kC;   // level 1 is largest
  return kgrad_coef_bytes(tr, Hq, n_queries) +
         static_cast<int64_t>(tr.B) * tr.Hkv * parents * kgrad_chunks(tr, n_queries) * kC * tr.d * 4;
}

int64_t kgrad_out_floats(const recsa_tree& tr) {
  int64_t n = 0;
  for (int l = 1; l < tr.n_levels; ++l)
    n += static_cast<int64_t>(tr.B) * tr.Hkv * level_rows_host(tr.L_cap, l) * tr.d;
  return n;
}

template <int DT, int D, int G>
static hipError_t kgrad_impl(const recsa_tree& tr, const void* q, int Hq, int T,
                             const int64_t* pos, const int32_t* sel, const int32_t* cnt,
                             const float* imp, const float* teacher, const float* logits,
                             float* dK, void* ws, hipStream_t s) {
  float* coef = static_cast<float*>(ws);
  const int64_t nq = static_cast<int64_t>(tr.B) * T;
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + kgrad_coef_bytes(tr, Hq, nq));
  const int n_chunks = static_cast<int>(kgrad_chunks(tr, nq));
  kgrad_coef_kernel<G><<<dim3(static_cast<unsigned>(nq), tr.Hkv), kBlock, 0, s>>>(
      tr, T, pos, sel, cnt, imp, teacher, logits, coef);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t off = 0;
  for (int l = 1; l < tr.n_levels; ++l) {
    const int64_t rows = level_rows_host(tr.L_cap, l);
    if (rows > 0) {
      const unsigned parents = static_cast<unsigned>((rows + kC - 1) / kC);
      dim3 ga(parents * n_chunks, tr.Hkv, tr.B);
      kgrad_accum_kernel<DT, D, G><<<ga, kBlock, 0, s>>>(tr, q, Hq, T, pos, sel, cnt, coef, l,
                                                         n_chunks, part);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      dim3 gf(parents, tr.Hkv, tr.B);
      kgrad_finish_kernel<D><<<gf, kBlock, 0, s>>>(tr, l, n_chunks, part, dK + off);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    off += static_cast<int64_t>(tr.B) * tr.Hkv * rows * D;
  }
  return hipSuccess;
}

hipError_t launch_kgrad(const recsa_tree& tr, const void* q, int Hq, int T, const int64_t* pos,
                        const int32_t* sel, const int32_t* cnt, const float* imp,
                        const float* teacher, const float* logits, float* dK, void* ws,
                        hipStream_t s) {
  RECSA_DISPATCH(kgrad_impl, tr, q, Hq, T, pos, sel, cnt, imp, teacher, logits, dK, ws, s);
}

}  // namespace recsa
