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
// kgrad_stats_kernel  per (query, KV head, scored level): each head's softmax
//                     figures (max, 1/Z, sum_f r_f P_h,f) from the selection
//                     logits, pi and y.
// kgrad_accum_kernel  per (sequence, KV head, level, chunk of 2048 queries,
//                     parent node w; XCD-contiguous): walks the chunk's
//                     queries in order, finds w among each query's parents,
//                     forms their coefficients for w's 16 children, and
//                     contracts coefficient x rotated query on the matrix
//                     cores.
// kgrad_finish_kernel per parent: the chunks in order, R(c)^T / sqrt(d), the
//                     rows out.  Fixed orders: identical bits on every call.
#include <math.h>

#include <algorithm>

#include "recsa_common.hpp"
#include "recsa_kernels.hpp"
#include "recsa_mfma.hpp"
#include "recsa_rope8.hpp"

namespace recsa {

namespace {

constexpr int kKgMatch = 8;        // matched queries per accumulation step
constexpr int kKgChunk = 2048;     // queries per accumulation workgroup
constexpr int kKgXcds = 8;         // XCDs the workgroups are dealt to

}  // namespace

// stats: [n_queries * Hkv][n_sel][G] of {max, 1/Z, sum_f r_f P_h,f, 0}, the
// softmax of each head's logits over a scored level's non-current candidates
// and its r-weighted mean.  One pass keeps each head's running (max, sum exp,
// sum r exp) for the thread's candidates; one block combine gives every
// head's figures.  The accumulation forms the coefficients from these.
template <int G>
__global__ void __launch_bounds__(kBlock) kgrad_stats_kernel(
    recsa_tree tr, int T, const int64_t* __restrict__ pos, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, const float* __restrict__ imp,
    const float* __restrict__ teacher, const float* __restrict__ logits,
    float4* __restrict__ stats) {
  constexpr int NW = kBlock / kWave;
  __shared__ float red[3 * G][NW];
  const int64_t qi = blockIdx.x;
  const int j = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wid = tid >> 6;
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
    const float* s = logits + base * G;
    float mx[G], z[G], w[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mx[h] = -INFINITY;
      z[h] = 0.f;
      w[h] = 0.f;
    }
    // hardware exp2 and reciprocal (about 1 ulp each), as the accumulation's
    // coefficient staging uses
    constexpr float kLog2e = 1.44269504088896341f;
    // four candidates per thread per step, 16-byte loads (a level's row of
    // C*k entries holds the reads past n; those lanes are skipped)
    for (int p0 = 4 * tid; p0 < n; p0 += 4 * kBlock) {
      const float4 y4 = *reinterpret_cast<const float4*>(yv + p0);
      const float4 p4 = *reinterpret_cast<const float4*>(pv + p0);
      const float ya[4] = {y4.x, y4.y, y4.z, y4.w};
      const float pa[4] = {p4.x, p4.y, p4.z, p4.w};
      float ra[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ra[e] = pa[e] > 0.f ? ya[e] * __builtin_amdgcn_rcpf(pa[e]) : 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float4 s4 = *reinterpret_cast<const float4*>(s + static_cast<int64_t>(h) * CK + p0);
        const float sa[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (p0 + e >= n) break;
          const float x = sa[e], r = ra[e];
          if (x > mx[h]) {
            const float sc = __builtin_amdgcn_exp2f((mx[h] - x) * kLog2e);
            z[h] = z[h] * sc + 1.f;
            w[h] = w[h] * sc + r;
            mx[h] = x;
          } else {
            const float ex = __builtin_amdgcn_exp2f((x - mx[h]) * kLog2e);
            z[h] += ex;
            w[h] += r * ex;
          }
        }
      }
    }
    // block combine: every head's max, then its rescaled sums
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float v = wave_max(mx[h]);
      if (lane == 0) red[h][wid] = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float m = red[h][0];
#pragma unroll
      for (int q = 1; q < NW; ++q) m = fmaxf(m, red[h][q]);
      const float sc = mx[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mx[h] - m) * kLog2e);
      mx[h] = m;
      z[h] *= sc;
      w[h] *= sc;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float zs = wave_sum(z[h]), ws = wave_sum(w[h]);
      if (lane == 0) {
        red[G + h][wid] = zs;
        red[2 * G + h][wid] = ws;
      }
    }
    __syncthreads();
    if (tid == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float zs = 0.f, ws = 0.f;
#pragma unroll
        for (int q = 0; q < NW; ++q) {
          zs += red[G + h][q];
          ws += red[2 * G + h][q];
        }
        const float inv = 1.0f / zs;
        stats[(slot * n_sel + (l - 1)) * G + h] = make_float4(mx[h], inv, ws * inv, 0.f);
      }
    }
    __syncthreads();                                 // red is reused by the next level
  }
}

// One workgroup per (parent node w of level l, chunk of kKgChunk queries) of
// one (sequence, KV head): the sum over the chunk's queries, in order, for
// w's children 16w .. 16w+15, before R(c)^T, into part[head][w][chunk][16][D].
// Workgroups of one XCD take consecutive (chunk, parent) ids, so those
// running together share one chunk's query rows in their L2.  Per batch of
// kKgMatch matched queries, the contraction
// coef[16 children][(m, h)] x q~[(m, h)][D] runs on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32, exact fp32 products, fp32 accumulation); wave wv
// owns the D/64 column tiles wv*D/64 ...
template <int DT, int D, int G>
__global__ void __launch_bounds__(kBlock) kgrad_accum_kernel(
    recsa_tree tr, const void* qv, int Hq, int T, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
    const float* __restrict__ imp, const float* __restrict__ teacher,
    const float* __restrict__ logits, const float4* __restrict__ stats, int level, int64_t n_par,
    int n_chunks, float* __restrict__ part) {
  using Ty = typename Stor<DT>::T;
  constexpr int H2 = D / 2;
  constexpr int TPW = D / 64;                        // 16-column tiles per wave
  constexpr int KB = kKgMatch * G;                   // contraction length per batch
  static_assert(KB % 4 == 0, "batch must fill whole 16x16x4 steps");
  constexpr int P8 = H2 / 8;                         // 8-pair items per query row
  __shared__ __attribute__((aligned(16))) float qt[KB][D];   // row m*G + h
  __shared__ __attribute__((aligned(16))) float cf[KB][kC];
  __shared__ int m_qi[kBlock], m_rho[kBlock], m_nv[kBlock], m_phi[kBlock];
  __shared__ int red_i[kBlock / kWave];
  // The device deals workgroups to its XCDs round-robin; renumber so that
  // each XCD takes one contiguous run of (chunk, parent) ids and its L2 holds
  // about one chunk's query rows at a time (placement only: any mapping is
  // correct).
  int64_t lin;
  {
    const int64_t nb = gridDim.x, bid = blockIdx.x;
    const int64_t x = bid % kKgXcds, per = nb / kKgXcds, extra = nb % kKgXcds;
    lin = x * per + min(x, extra) + bid / kKgXcds;
  }
  const int64_t w = lin % n_par;
  lin /= n_par;
  const int chunk = static_cast<int>(lin % n_chunks);
  lin /= n_chunks;
  const int j = static_cast<int>(lin % tr.Hkv), b = static_cast<int>(lin / tr.Hkv);
  const int64_t q_lo = static_cast<int64_t>(b) * T + static_cast<int64_t>(chunk) * kKgChunk;
  const int64_t q_hi = min(q_lo + kKgChunk, static_cast<int64_t>(b + 1) * T);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int n_sel = tr.n_levels - 1, k = tr.k, CK = kC * k, top = tr.n_levels - 1;
  f32x4_t acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

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
      // rotated, rounded query rows q~ = rnd(R(phi) q_h), 8 RoPE pairs per
      // item; zero past mc
      for (int item = tid; item < KB * P8; item += kBlock) {
        const int row = item / P8, j0 = 8 * (item % P8);
        const int m = row / G, h = row % G;
        float xo[8], yo[8];
        if (m < mc) {
          const int64_t qq = q0 + m_qi[m0 + m];
          const Ty* qr = static_cast<const Ty*>(qv) + (qq * Hq + static_cast<int64_t>(j) * G + h) * D;
          rotate8_pairs<DT, D>(qr, j0, tr.rope + static_cast<int64_t>(m_phi[m0 + m]) * H2 * 2, xo,
                               yo);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xo[e] = Stor<DT>::round(xo[e]);
            yo[e] = Stor<DT>::round(yo[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xo[e] = yo[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
          *reinterpret_cast<float4*>(&qt[row][j0 + e]) =
              make_float4(xo[e], xo[e + 1], xo[e + 2], xo[e + 3]);
          *reinterpret_cast<float4*>(&qt[row][H2 + j0 + e]) =
              make_float4(yo[e], yo[e + 1], yo[e + 2], yo[e + 3]);
        }
      }
      // coefficients d KL / d s = -(P / G)(r - sum_f r_f P_f), four children
      // per item, from the logits, pi, y and the head's softmax figures (the
      // row's 16 slots lie inside its C*k entries; slots past nv are zeroed)
      for (int item = tid; item < KB * (kC / 4); item += kBlock) {
        const int row = item / (kC / 4), c0 = 4 * (item % (kC / 4));
        const int m = row / G, h = row % G;
        float cv[4] = {0.f, 0.f, 0.f, 0.f};
        if (m < mc) {
          const int nvm = m_nv[m0 + m];
          if (c0 < nvm) {
            const int64_t lrow = ((q0 + m_qi[m0 + m]) * tr.Hkv + j) * n_sel + (level - 1);
            const int64_t off = kC * m_rho[m0 + m] + c0;
            const float4 st = stats[lrow * G + h];
            const float4 s4 = *reinterpret_cast<const float4*>(
                logits + (lrow * G + h) * static_cast<int64_t>(CK) + off);
            const float4 y4 = *reinterpret_cast<const float4*>(teacher + lrow * CK + off);
            const float4 p4 = *reinterpret_cast<const float4*>(imp + lrow * CK + off);
            const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
            const float yv[4] = {y4.x, y4.y, y4.z, y4.w};
            const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
            // hardware exp2 and reciprocal (about 1 ulp each): this staging
            // runs once per (query, parent, head) on the accumulation's path
            constexpr float kLog2e = 1.44269504088896341f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (c0 + e < nvm) {
                const float r = pv[e] > 0.f ? yv[e] * __builtin_amdgcn_rcpf(pv[e]) : 0.f;
                const float P = __builtin_amdgcn_exp2f((sv[e] - st.x) * kLog2e) * st.y;
                cv[e] = -(P * (1.0f / G)) * (r - st.z);
              }
            }
          }
        }
        *reinterpret_cast<float4*>(&cf[row][c0]) = make_float4(cv[0], cv[1], cv[2], cv[3]);
      }
      __syncthreads();
      // A[child][kk] = cf[kk][child], B[kk][col] = qt[kk][col], kk = 4s + lane/16
      const int ks = (mc * G + 3) / 4;
      for (int st = 0; st < ks; ++st) {
        const int kk = 4 * st + (lane >> 4);
        const float a = cf[kk][lane & 15];
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const float bv = qt[kk][(wv * TPW + u) * 16 + (lane & 15)];
          acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc[u], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }
  float* pp = part + (((static_cast<int64_t>(b) * tr.Hkv + j) * n_par + w) * n_chunks + chunk) *
                         (kC * D);
  // C[row 4*(lane/16) + r][column lane % 16] of each tile
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      pp[(4 * (lane >> 4) + r) * D + (wv * TPW + u) * 16 + (lane & 15)] = acc[u][r];
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
// Workspace: the softmax figures [n_queries*Hkv][n_sel][G] (float4), then
// the chunk sums of the largest level, [B*Hkv][parents][chunks][16][d].
static int64_t kgrad_stats_bytes(const recsa_tree& tr, int Hq, int64_t n_queries) {
  const int n_sel = tr.n_levels > 1 ? tr.n_levels - 1 : 1;
  return align256(n_queries * tr.Hkv * n_sel * static_cast<int64_t>(Hq / tr.Hkv) * 16);
}

static int64_t kgrad_chunks(const recsa_tree& tr, int64_t n_queries) {
  const int64_t T = n_queries / tr.B;
  return (T + kKgChunk - 1) / kKgChunk;
}

int64_t kgrad_ws_bytes(const recsa_tree& tr, int Hq, int64_t n_queries) {
  const int64_t parents = (level_rows_host(tr.L_cap, 1) + kC - 1) / kC;   // level 1 is largest
  return kgrad_stats_bytes(tr, Hq, n_queries) +
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
  float4* stats = static_cast<float4*>(ws);
  const int64_t nq = static_cast<int64_t>(tr.B) * T;
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + kgrad_stats_bytes(tr, Hq, nq));
  const int n_chunks = static_cast<int>(kgrad_chunks(tr, nq));
  kgrad_stats_kernel<G><<<dim3(static_cast<unsigned>(nq), tr.Hkv), kBlock, 0, s>>>(
      tr, T, pos, sel, cnt, imp, teacher, logits, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t off = 0;
  for (int l = 1; l < tr.n_levels; ++l) {
    const int64_t rows = level_rows_host(tr.L_cap, l);
    if (rows > 0) {
      const unsigned parents = static_cast<unsigned>((rows + kC - 1) / kC);
      const int64_t n_wg = static_cast<int64_t>(parents) * n_chunks * tr.Hkv * tr.B;
      if (n_wg > 0x7fffffff) return hipErrorInvalidConfiguration;
      kgrad_accum_kernel<DT, D, G><<<dim3(static_cast<unsigned>(n_wg)), kBlock, 0, s>>>(
          tr, q, Hq, T, pos, sel, cnt, imp, teacher, logits, stats, l, parents, n_chunks, part);
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
