// Pooler distillation losses (picx.dev Pooler Distillation, Eq. 6 and Eq. 7).
//
// Eq. 6 compares, per query and scored level, the student importance pi (the
// walk's head-mean softmax over the non-current candidates, as recsa_select
// reports it) with the teacher's subtree mass y: the dense causal attention
// of the same query heads over the tokens [0, t], at the true RoPE positions,
// summed over each candidate's subtree and renormalised over the candidates.
//
// The teacher is computed in two launches:
//   teacher_lse_kernel  one pass over the keys of a block of queries with
//                       split-bf16 matrix-core products (float32-level
//                       accuracy); a 16x16 output tile is one level-1 group of
//                       16 tokens against 16 (query, head) rows, so each tile
//                       reduces to the group's log-sum-exp per row, which does
//                       not depend on the row's global maximum: no second pass.
//   distill_kl_kernel   per (query, KV head): the softmax normaliser from the
//                       group log-sum-exps, the head-mean mass of every level-1
//                       group, the candidates' subtree masses at each scored
//                       level, and KL(y || pi).
// Eq. 7 reruns the pooler on every complete node (pool_tile in its statistics
// mode), writes per-tile sums and reduces them in a fixed order.
#include <math.h>

#include <algorithm>

#include "recsa_common.hpp"
#include "recsa_kernels.hpp"
#include "recsa_mfma.hpp"
#include "recsa_pool.hpp"
#include "recsa_rope8.hpp"

namespace recsa {

namespace {

constexpr int kTeacherSets = 3;    // 16-row query sets per teacher wave
constexpr int kTeacherRows = 16 * kTeacherSets * (kBlock / kWave);   // rows per workgroup
constexpr int kTeacherKeys = 64;   // keys per tile: four level-1 groups

// The G log-sum-exps of one level-1 group (consecutive floats).
template <int G>
__device__ __forceinline__ void load_group(const float* p, float* x) {
  if constexpr (G == 4) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x;
    x[1] = v.y;
    x[2] = v.z;
    x[3] = v.w;
  } else if constexpr (G == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    x[0] = v.x;
    x[1] = v.y;
  } else {
    x[0] = *p;
  }
}

__device__ __forceinline__ float block_sum(float v, float* red) {
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

// ------------------------------------------------------------ teacher
// Workgroup: kTeacherRows/G consecutive queries of one (sequence, KV head),
// i.e. kTeacherRows = 16 kTeacherSets x 4 rows r = G*(query - first) + h;
// wave w owns the kTeacherSets sets of 16 rows starting at 16 kTeacherSets w.
// Logits on the bf16 matrix cores at float32-level accuracy: every rotated
// float32 operand x is split into x_hi = rnd(x) and x_lo = rnd(x - x_hi)
// (bf16; |x - x_hi - x_lo| <= 2^-18 |x|), and each 32-dim block takes the
// products lo.hi + hi.lo + hi.hi; the dropped lo.lo term and the split
// residuals stay below 4 * 2^-18 of each product (float32 accumulation of
// d = 128 products carries a similar bound).  v_mfma_f32_16x16x32_bf16 runs
// with the keys as the A operand and the wave's 16 query rows as B, so one
// 16 x 16 tile is one level-1 group (rows) against 16 query rows (columns)
// and lane l holds 4 keys of column l % 16: a row's log-sum-exp over the
// group reduces 4 registers and the 4 lanes l % 16 + 16 i.  The group's
// log-sum-exp does not depend on the row's global maximum: one pass.
// Every key row is rotated at its absolute position and split once for the
// whole call (teacher_keys_kernel); each tile of 64 keys is then staged into
// LDS with 16-byte loads by all 256 threads.
// lse: [B*T][Hkv][ng_cap][G] float32 group log-sum-exps in base-2 units
// (log2 of the sum of 2^(logit log2 e)); entry (v, h) is written for every
// level-1 group v <= t/16 of the row's query, never beyond.
// Every level-0 key row rotated at its absolute position and split once:
// ksplit[b][j][tau] = {hi[D], lo[D]} (bf16), each thread 8 RoPE pairs of one
// row.  The key tiles of every query block are then plain 16-byte loads.
template <int DT, int D>
__global__ void __launch_bounds__(kBlock) teacher_keys_kernel(recsa_tree tr,
                                                              const float* __restrict__ arope,
                                                              uint16_t* __restrict__ ksplit) {
  using Ty = typename Stor<DT>::T;
  constexpr int H2 = D / 2;
  constexpr int TPR = H2 / 8;                     // threads per row
  constexpr int RPB = kBlock / TPR;               // rows per workgroup
  const int64_t tau = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
  if (tau >= tr.L_cap) return;
  const int j0 = 8 * (threadIdx.x % TPR);
  const int64_t head = static_cast<int64_t>(blockIdx.z) * tr.Hkv + blockIdx.y;
  const Ty* row = static_cast<const Ty*>(tr.K[0]) + (head * tr.L_cap + tau) * D;
  float xo[8], yo[8];
  rotate8_pairs<DT, D>(row, j0, arope + tau * H2 * 2, xo, yo);
  uint4 xh, xl, yh, yl;
  split_bf16x8(xo, xh, xl);
  split_bf16x8(yo, yh, yl);
  uint16_t* dst = ksplit + (head * tr.L_cap + tau) * 2 * D;
  *reinterpret_cast<uint4*>(dst + j0) = xh;
  *reinterpret_cast<uint4*>(dst + H2 + j0) = yh;
  *reinterpret_cast<uint4*>(dst + D + j0) = xl;
  *reinterpret_cast<uint4*>(dst + D + H2 + j0) = yl;
}

// One staged key tile (kTeacherKeys keys = four level-1 groups) against a
// wave's kTeacherSets sets of 16 query columns: per group, the 16x16 logits of
// each set on the matrix cores (split products lo.hi + hi.lo + hi.hi; each key
// fragment read from LDS once for all sets), then per column the group's
// log-sum-exp, stored in base-2 units.  MASK applies causality (keys
// after the column's position drop out); without it every key counts.
template <bool MASK, int D, int G>
__device__ __forceinline__ void teacher_tile_lse(const uint16_t (*khi)[D + 8],
                                                 const uint16_t (*klo)[D + 8],
                                                 const uint4 (*bhi)[D / 32],
                                                 const uint4 (*blo)[D / 32], int tau0, int tmax,
                                                 const int* t_col, int col, int hh, float scale2,
                                                 float* const* lcol) {
  constexpr int KB = D / 32;
  constexpr int NS = kTeacherSets;
#pragma unroll
  for (int g = 0; g < kTeacherKeys / kC; ++g) {
    const int tg = tau0 + kC * g;   // first token of the level-1 group
    if (MASK && tg > tmax) break;   // uniform
    f32x4_t acc[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint4 ah = *reinterpret_cast<const uint4*>(&khi[kC * g + col][32 * kb + 8 * hh]);
      const uint4 al = *reinterpret_cast<const uint4*>(&klo[kC * g + col][32 * kb + 8 * hh]);
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al),
                                                         __builtin_bit_cast(bf16x8_t, bhi[u][kb]),
                                                         acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                         __builtin_bit_cast(bf16x8_t, blo[u][kb]),
                                                         acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                         __builtin_bit_cast(bf16x8_t, bhi[u][kb]),
                                                         acc[u], 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      // keys tg + 4 hh + i against the query of column `col`, base-2 logits
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = acc[u][i] * scale2;
        if (MASK && tg + 4 * hh + i > t_col[u]) sv[i] = -INFINITY;
      }
      float m = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      // exp2(-inf) = 0 drops masked keys; a column with no key left has
      // m = -inf and stores nothing
      float e = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) e += __builtin_amdgcn_exp2f(sv[i] - m);
      e += __shfl_xor(e, 16);
      e += __shfl_xor(e, 32);
      if (hh == 0 && t_col[u] >= 0 && (!MASK || m != -INFINITY))
        lcol[u][static_cast<int64_t>(tg >> 4) * G] = m + __builtin_amdgcn_logf(e);
    }
  }
}

template <int DT, int D, int G>
__global__ void __launch_bounds__(kBlock) teacher_lse_kernel(recsa_tree tr, const void* qv,
                                                             int T, const int64_t* __restrict__ pos,
                                                             const float* __restrict__ arope,
                                                             const uint16_t* __restrict__ ksplit,
                                                             float* __restrict__ lse, int ng_cap) {
  using Ty = typename Stor<DT>::T;
  constexpr int QB = kTeacherRows / G;
  constexpr int H2 = D / 2;
  constexpr int KB = D / 32;             // 32-dim blocks
  constexpr int LDK = D + 8;             // bf16 elements per LDS key row (16-byte aligned)
  constexpr int DQ = D / 4;              // dims per thread per key row in a tile load
  __shared__ __attribute__((aligned(16))) uint16_t khi[kTeacherKeys][LDK];
  __shared__ __attribute__((aligned(16))) uint16_t klo[kTeacherKeys][LDK];
  __shared__ int st[kTeacherRows];
  __shared__ int s_tmax, s_tmin;
  const int j = blockIdx.y, b = blockIdx.z;
  // longest query blocks first: causal work grows with the position
  const int q0 = (gridDim.x - 1 - blockIdx.x) * QB;
  const int Hq = tr.Hkv * G;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid >> 6;
  const int col = lane & 15, hh = lane >> 4;

  if (tid < kTeacherRows) {
    const int qi = q0 + tid / G;
    st[tid] = qi < T ? static_cast<int>(pos[static_cast<int64_t>(b) * T + qi]) : -1;
  }
  __syncthreads();
  if (wid == 0) {
    static_assert(kTeacherRows % kWave == 0, "rows fill whole waves");
    float m = -1.f, mn = 3.0e7f;
#pragma unroll
    for (int r = lane; r < kTeacherRows; r += kWave) {
      const int t = st[r];
      m = fmaxf(m, static_cast<float>(t));
      if (t >= 0) mn = fminf(mn, static_cast<float>(t));
    }
    m = wave_max(m);
    mn = -wave_max(-mn);
    if (lane == 0) {
      s_tmax = static_cast<int>(m);
      s_tmin = static_cast<int>(mn);
    }
  }
  // B operand: this wave's kTeacherSets x 16 query rows R(t) q, split; lane
  // holds column `col` of each set, dims 32 kb + 8 hh + [0, 8) (both members
  // of each RoPE pair)
  constexpr int NS = kTeacherSets;
  int t_col[NS];
  float* lcol[NS];
  uint4 bhi[NS][KB], blo[NS][KB];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int r_col = 16 * (NS * wid + u) + col;
    t_col[u] = st[r_col];
    const int qi = min(q0 + r_col / G, T - 1), h = r_col % G;
    lcol[u] = lse + ((static_cast<int64_t>(b) * T + qi) * tr.Hkv + j) * ng_cap * G + h;
    const Ty* qr =
        static_cast<const Ty*>(qv) + ((static_cast<int64_t>(b) * T + qi) * Hq + j * G + h) * D;
#pragma unroll
    for (int kb = 0; kb < KB / 2; ++kb) {
      float xo[8], yo[8];
      if (t_col[u] >= 0) {
        rotate8_pairs<DT, D>(qr, 32 * kb + 8 * hh,
                           arope + static_cast<int64_t>(t_col[u]) * H2 * 2, xo, yo);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xo[e] = yo[e] = 0.f;
      }
      split_bf16x8(xo, bhi[u][kb], blo[u][kb]);
      split_bf16x8(yo, bhi[u][kb + KB / 2], blo[u][kb + KB / 2]);
    }
  }
  __syncthreads();
  const int tmax = s_tmax, tmin = s_tmin;
  if (tmax < 0) return;   // no query in this block (uniform)
  const uint16_t* ks = ksplit + (static_cast<int64_t>(b) * tr.Hkv + j) * tr.L_cap * 2 * D;
  // logits in base-2 units: log2(e) / sqrt(d) folded into the scale, so each
  // exponential and the final logarithm are single hardware instructions
  const float scale2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(D)));
  const int kk = tid >> 2, qq = tid & 3;     // the key row and quarter this thread loads

  // each tile's rows pass through registers into LDS (three row sets per
  // wave leave no registers for fetching the next tile ahead)
  uint4 ph[DQ / 8], pl[DQ / 8];
  auto fetch = [&](int tau0) {
    const int tau = tau0 + kk;
    const uint16_t* src = ks + static_cast<int64_t>(tau) * 2 * D + qq * DQ;
#pragma unroll
    for (int c = 0; c < DQ / 8; ++c) {
      ph[c] = make_uint4(0u, 0u, 0u, 0u);
      pl[c] = ph[c];
      if (tau <= tmax) {
        ph[c] = *reinterpret_cast<const uint4*>(src + 8 * c);
        pl[c] = *reinterpret_cast<const uint4*>(src + D + 8 * c);
      }
    }
  };
  const int n_tiles = tmax / kTeacherKeys + 1;
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int tau0 = tile * kTeacherKeys;
    __syncthreads();   // the previous tile is read
    fetch(tau0);
#pragma unroll
    for (int c = 0; c < DQ / 8; ++c) {
      *reinterpret_cast<uint4*>(&khi[kk][qq * DQ + 8 * c]) = ph[c];
      *reinterpret_cast<uint4*>(&klo[kk][qq * DQ + 8 * c]) = pl[c];
    }
    __syncthreads();
    // tiles wholly at or before every query of the block need no causal mask
    if (tau0 + kTeacherKeys - 1 <= tmin)
      teacher_tile_lse<false, D, G>(khi, klo, bhi, blo, tau0, tmax, t_col, col, hh, scale2, lcol);
    else
      teacher_tile_lse<true, D, G>(khi, klo, bhi, blo, tau0, tmax, t_col, col, hh, scale2, lcol);
  }
}

// ------------------------------------------------------------ Eq. 6 terms
// One workgroup per (query, KV head).  Dynamic LDS: m1[ng_cap] (head-mean
// teacher mass of each level-1 group), mass[C*k], red[32].
template <int G>
__global__ void __launch_bounds__(kBlock) distill_kl_kernel(
    recsa_tree tr, int T, const int64_t* __restrict__ pos, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, const float* __restrict__ imp,
    const float* __restrict__ lse, int ng_cap, float* __restrict__ kl, float* __restrict__ yout) {
  extern __shared__ float dsm[];
  const int qi = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t slot = (static_cast<int64_t>(b) * T + qi) * tr.Hkv + j;
  const int n_sel = tr.n_levels - 1, k = tr.k, CK = kC * k, top = tr.n_levels - 1;
  const int64_t t = pos[static_cast<int64_t>(b) * T + qi];
  const int ng = static_cast<int>(t >> 4) + 1;
  const float* L = lse + slot * ng_cap * G;
  float* m1 = dsm;
  float* mass = dsm + ng_cap;
  float* red = mass + CK;

  // softmax normaliser of each head, log2 Z_h = log2-sum-exp2 over the
  // groups (the group figures are in base-2 units, so every exponential and
  // logarithm is one hardware instruction): one pass of G-wide loads with a
  // running (max, sum) per head, then one block exchange for all heads
  float mx[G], sx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mx[h] = -INFINITY;
    sx[h] = 0.f;
  }
  for (int v = tid; v < ng; v += kBlock) {
    float x[G];
    load_group<G>(L + static_cast<int64_t>(v) * G, x);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (x[h] > mx[h]) {
        sx[h] = sx[h] * __builtin_amdgcn_exp2f(mx[h] - x[h]) + 1.0f;   // 2^-inf = 0 at first
        mx[h] = x[h];
      } else {
        sx[h] += __builtin_amdgcn_exp2f(x[h] - mx[h]);
      }
    }
  }
  float lz[G];
  {
    const int lane = tid & (kWave - 1), wid = tid >> 6;
    float* rm = red;               // [G][4] wave maxima, then [G][4] wave sums
    float* rs = red + 4 * G;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float wm = wave_max(mx[h]);
      const float ws =
          wave_sum(mx[h] == -INFINITY ? 0.f : sx[h] * __builtin_amdgcn_exp2f(mx[h] - wm));
      if (lane == 0) {
        rm[4 * h + wid] = wm;
        rs[4 * h + wid] = ws;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float m = rm[4 * h];
#pragma unroll
      for (int w = 1; w < kBlock / kWave; ++w) m = fmaxf(m, rm[4 * h + w]);
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kBlock / kWave; ++w)
        sum += rm[4 * h + w] == -INFINITY
                   ? 0.f
                   : rs[4 * h + w] * __builtin_amdgcn_exp2f(rm[4 * h + w] - m);
      lz[h] = m + __builtin_amdgcn_logf(sum);
    }
  }
  for (int v = tid; v < ng; v += kBlock) {
    float x[G];
    load_group<G>(L + static_cast<int64_t>(v) * G, x);
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) s += __builtin_amdgcn_exp2f(x[h] - lz[h]);
    m1[v] = s * (1.0f / G);
  }
  __syncthreads();

  const int32_t* sl = sel + slot * n_sel * k;
  const int32_t* cl = cnt + slot * n_sel;
  const float* il = imp + slot * n_sel * CK;
  float* ko = kl + slot * n_sel;
  float* yo = yout ? yout + slot * n_sel * CK : nullptr;
  for (int l = 1; l <= n_sel; ++l) {
    const ListView lv = list_view(t, l, top, k, sl, cl);
    if (lv.len <= k) {   // unscored (uniform)
      if (tid == 0) ko[l - 1] = 0.f;
      if (yo)
        for (int p = tid; p < CK; p += kBlock) yo[static_cast<int64_t>(l - 1) * CK + p] = 0.f;
      continue;
    }
    const int n_oth = lv.len - 1;
    const int64_t span = int64_t{1} << (4 * (l - 1));   // level-1 groups under a level-l node
    float part = 0.f;
    for (int p = tid; p < n_oth; p += kBlock) {
      const int64_t u = lv.node(p);
      const int64_t lo = u * span, hi = min((u + 1) * span, static_cast<int64_t>(ng));
      float s = 0.f;
      for (int64_t v = lo; v < hi; ++v) s += m1[v];
      mass[p] = s;
      part += s;
    }
    const float tot = block_sum(part, red);
    float acc = 0.f;
    for (int p = tid; p < n_oth; p += kBlock) {
      const float y = mass[p] / tot;
      if (y > 0.f) acc += y * (logf(y) - logf(il[static_cast<int64_t>(l - 1) * CK + p]));
    }
    if (yo)
      for (int p = tid; p < CK; p += kBlock)
        yo[static_cast<int64_t>(l - 1) * CK + p] = p < n_oth ? mass[p] / tot : 0.f;
    const float v = block_sum(acc, red);
    if (tid == 0) ko[l - 1] = v;
  }
}

// ------------------------------------------------------------ Eq. 7
// Per level: one workgroup per tile of 16 complete nodes of one (sequence,
// KV head); partial row [D + 1] = (sum of sigma*m, sum of ||mu||^2).
template <int DT, int D>
__global__ void __launch_bounds__(kBlock) shift_stats_kernel(recsa_tree tr, recsa_pooler P,
                                                             int level, int64_t n_nodes,
                                                             float* __restrict__ part) {
  using Ty = typename Stor<DT>::T;
  constexpr int NODES = 16;
  __shared__ PoolSmem<DT, D, NODES> sm;
  const int j = blockIdx.y, b = blockIdx.z;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * NODES;
  const int n_valid = static_cast<int>(min<int64_t>(NODES, n_nodes - first));
  const int64_t rows_up = level_rows_dev(tr.L_cap, level - 1);
  const int64_t head = static_cast<int64_t>(b) * tr.Hkv + j;
  const Ty* kc = static_cast<const Ty*>(tr.K[level - 1]) + (head * rows_up + first * kC) * D;
  float* out = part + (head * gridDim.x + blockIdx.x) * (D + 1);
  pool_tile<DT, D, NODES, kBlock, true>(kc, nullptr, nullptr, nullptr, nullptr, 0, nullptr,
                                        n_valid, P, sm, out);
}

struct ShiftLevels {
  int64_t part_off[RECSA_MAX_LEVELS];   // floats
  int64_t n_rows[RECSA_MAX_LEVELS];     // partial rows (tiles * heads)
  int64_t n_nodes[RECSA_MAX_LEVELS];    // complete nodes, all heads
};

// One workgroup per level >= 1: sums the partial rows in a fixed order
// (four row groups of 64 columns each, float64), then the penalty
// ||sum sigma m||^2 / (M * sum ||mu||^2) = ||mean sigma m||^2 / mean ||mu||^2.
template <int D>
__global__ void __launch_bounds__(kBlock) shift_reduce_kernel(const float* __restrict__ part,
                                                              ShiftLevels lv,
                                                              float* __restrict__ out) {
  constexpr int NCOL = D + 1;
  constexpr int NCB = (NCOL + kWave - 1) / kWave;
  __shared__ double acc_s[kBlock / kWave][NCB * kWave];
  __shared__ double s_num;
  const int l = blockIdx.x + 1;
  const int lane = threadIdx.x & (kWave - 1), rg = threadIdx.x >> 6;
  const float* base = part + lv.part_off[l];
  const int64_t n_rows = lv.n_rows[l];
  double acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = 0.0;
  for (int64_t r = rg; r < n_rows; r += kBlock / kWave) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = cb * kWave + lane;
      if (c < NCOL) acc[cb] += static_cast<double>(base[r * NCOL + c]);
    }
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc_s[rg][cb * kWave + lane] = acc[cb];
  __syncthreads();
  float* o = out + static_cast<int64_t>(l - 1) * (D + 2);
  if (threadIdx.x < kWave) {
    double num = 0.0;
    for (int c = lane; c < NCOL; c += kWave) {
      double s = 0.0;
      for (int g = 0; g < kBlock / kWave; ++g) s += acc_s[g][c];
      o[c] = static_cast<float>(s);
      if (c < D) num += s * s;
      acc_s[0][c] = s;
    }
    for (int off = kWave / 2; off > 0; off >>= 1) num += __shfl_xor(num, off);
    if (lane == 0) s_num = num;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double m = static_cast<double>(lv.n_nodes[l]);
    const double den = m * acc_s[0][D];
    o[D + 1] = (lv.n_nodes[l] > 0 && den > 0.0) ? static_cast<float>(s_num / den) : 0.f;
  }
}

// ------------------------------------------------------------ launchers
int64_t distill_groups(int64_t L_cap) { return (L_cap + kC - 1) / kC; }

template <int DT, int D, int G>
static hipError_t distill_impl(const recsa_tree& tr, const void* q, int Hq, int T,
                               const int64_t* pos, const int32_t* sel, const int32_t* cnt,
                               const float* imp, double theta, float* kl, float* y, void* ws,
                               hipStream_t s) {
  (void)Hq;
  float* arope = static_cast<float*>(ws);
  const int64_t rope_bytes = align256(tr.L_cap * D * 4);
  uint16_t* ksplit = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + rope_bytes);
  const int64_t ks_bytes = align256(static_cast<int64_t>(tr.B) * tr.Hkv * tr.L_cap * D * 4);
  float* lse = reinterpret_cast<float*>(static_cast<char*>(ws) + rope_bytes + ks_bytes);
  const int ng_cap = static_cast<int>(distill_groups(tr.L_cap));
  hipError_t e = launch_rope_table(arope, D, static_cast<int>(tr.L_cap), theta, s);
  if (e != hipSuccess) return e;
  {
    constexpr int RPB = kBlock / (D / 16);
    dim3 gk(static_cast<unsigned>((tr.L_cap + RPB - 1) / RPB), tr.Hkv, tr.B);
    teacher_keys_kernel<DT, D><<<gk, kBlock, 0, s>>>(tr, arope, ksplit);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr int QB = kTeacherRows / G;
  dim3 g1(static_cast<unsigned>((T + QB - 1) / QB), tr.Hkv, tr.B);
  teacher_lse_kernel<DT, D, G><<<g1, kBlock, 0, s>>>(tr, q, T, pos, arope, ksplit, lse, ng_cap);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(static_cast<unsigned>(T), tr.Hkv, tr.B);
  const size_t lds = (static_cast<size_t>(ng_cap) + kC * tr.k + 32) * sizeof(float);
  distill_kl_kernel<G><<<g2, kBlock, lds, s>>>(tr, T, pos, sel, cnt, imp, lse, ng_cap, kl, y);
  return hipGetLastError();
}

int64_t distill_ws_bytes(const recsa_tree& tr, int Hq, int64_t n_queries) {
  return align256(tr.L_cap * tr.d * 4) +
         align256(static_cast<int64_t>(tr.B) * tr.Hkv * tr.L_cap * tr.d * 4) +
         n_queries * Hq * distill_groups(tr.L_cap) * 4;
}

hipError_t launch_distill_kl(const recsa_tree& tr, const void* q, int Hq, int T,
                             const int64_t* pos, const int32_t* sel, const int32_t* cnt,
                             const float* imp, double theta, float* kl, float* y, void* ws,
                             hipStream_t s) {
  RECSA_DISPATCH(distill_impl, tr, q, Hq, T, pos, sel, cnt, imp, theta, kl, y, ws, s);
}

static ShiftLevels shift_levels(const recsa_tree& tr, int64_t tok_end) {
  ShiftLevels lv{};
  const int64_t heads = static_cast<int64_t>(tr.B) * tr.Hkv;
  int64_t off = 0;
  for (int l = 1; l < tr.n_levels; ++l) {
    const int64_t cap_tiles = (level_rows_host(tr.L_cap, l) + 15) / 16;
    const int64_t n = std::min(tok_end >> (4 * l), level_rows_host(tr.L_cap, l));
    lv.part_off[l] = off;
    lv.n_rows[l] = (n + 15) / 16 * heads;
    lv.n_nodes[l] = n * heads;
    off += cap_tiles * heads * (tr.d + 1);
  }
  lv.part_off[0] = off;   // total floats
  return lv;
}

int64_t shift_ws_bytes(const recsa_tree& tr) {
  return shift_levels(tr, tr.L_cap).part_off[0] * 4;
}

template <int DT, int D>
static hipError_t shift_impl(const recsa_tree& tr, const recsa_pooler& P, int64_t tok_end,
                             float* out, void* ws, hipStream_t s) {
  const ShiftLevels lv = shift_levels(tr, tok_end);
  float* part = static_cast<float*>(ws);
  for (int l = 1; l < tr.n_levels; ++l) {
    const int64_t n = lv.n_nodes[l] / (static_cast<int64_t>(tr.B) * tr.Hkv);
    if (n == 0) continue;
    dim3 grid(static_cast<unsigned>((n + 15) / 16), tr.Hkv, tr.B);
    shift_stats_kernel<DT, D><<<grid, kBlock, 0, s>>>(tr, P, l, n, part + lv.part_off[l]);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  shift_reduce_kernel<D><<<tr.n_levels - 1, kBlock, 0, s>>>(part, lv, out);
  return hipGetLastError();
}

hipError_t launch_shift_penalty(const recsa_tree& tr, const recsa_pooler& P, int64_t tok_end,
                                float* out, void* ws, hipStream_t s) {
  if (tr.dtype == RECSA_BF16)
    return tr.d == 128 ? shift_impl<RECSA_BF16, 128>(tr, P, tok_end, out, ws, s)
                       : shift_impl<RECSA_BF16, 64>(tr, P, tok_end, out, ws, s);
  return tr.d == 128 ? shift_impl<RECSA_F32, 128>(tr, P, tok_end, out, ws, s)
                     : shift_impl<RECSA_F32, 64>(tr, P, tok_end, out, ws, s);
}

}  // namespace recsa
