// Hierarchical selection (picx.dev Hierarchical Selection, Eq. 3) and the
// unified softmax (Unified Softmax, Eq. 4) with candidate-local RoPE (Key
// Theoretical Insight), split so that keys turn by their in-group offset and
// queries by the group distance ("slot-based rotation splitting", Conclusion).
//
// Per level l (top-down) two kernels run:
//   score_kernel  -- logits of every non-current candidate of A^(l) for the G
//                    query heads of one KV head, 256 list positions per
//                    workgroup; written to the workspace.
//   topk_kernel   -- importance (head-mean softmax), exact top-(k-1) by LDS
//                    radix select with lowest-index ties, S^(l) in ascending
//                    order plus a bitmap of selected list positions.
// Then attn_kernel gathers level-0 tokens (logits computed on the fly) and
// the unselected summaries (logits reused), with an online softmax over
// 256-position chunks; combine_kernel merges the decode chunks.
#include "recsa_common.hpp"
#include "recsa_kernels.hpp"

namespace recsa {

// ------------------------------------------------------------------------
// Logits of the 16 rows of one list group against G rotated query heads.
// Lane = (row c = lane/4, quarter s = lane%4); each lane rotates 2*E pairs of
// its row by the in-group offset c, rounds them to the storage dtype and dots
// them with the group's rotated query (LDS, float).  The four quarter lanes
// of a row are then summed, so every lane of row c ends with its G logits.
template <int DT, int D, int G>
__device__ __forceinline__ void group_logits(const typename Stor<DT>::T* __restrict__ rows,
                                             int nvalid, const float* qt,
                                             const float* __restrict__ rope, float* lg) {
  constexpr int E = D / 16, QD = D / 4, H2 = D / 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane >> 2, s = lane & 3;
  float acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.f;
  if (c < nvalid) {
    const typename Stor<DT>::T* row = rows + static_cast<int64_t>(c) * D;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int base = hh * QD + s * E;
      float x[E], y[E];
      load_vec<DT, E>(row + base, x);
      load_vec<DT, E>(row + H2 + base, y);
      const float* rp = rope + (c * H2 + base) * 2;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        float xo, yo;
        rope_pair(x[m], y[m], rp[2 * m], rp[2 * m + 1], xo, yo);
        xo = Stor<DT>::round(xo);
        yo = Stor<DT>::round(yo);
#pragma unroll
        for (int g = 0; g < G; ++g)
          acc[g] += qt[g * D + base + m] * xo + qt[g * D + H2 + base + m] * yo;
      }
    }
  }
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = acc[g];
    v += __shfl_xor(v, 1, kWave);
    v += __shfl_xor(v, 2, kWave);
    lg[g] = v * scale;
  }
}

// Rotate the G query heads by phi and round (one wave): qt = rnd(R(phi) q).
template <int DT, int D, int G>
__device__ __forceinline__ void rotate_query(const float* qs, float* qt, int phi,
                                             const float* __restrict__ rope) {
  constexpr int H2 = D / 2;
  const int lane = threadIdx.x & (kWave - 1);
  for (int idx = lane; idx < G * H2; idx += kWave) {
    const int g = idx / H2, j = idx % H2;
    const float* rp = rope + (static_cast<int64_t>(phi) * H2 + j) * 2;
    float xo, yo;
    rope_pair(qs[g * D + j], qs[g * D + j + H2], rp[0], rp[1], xo, yo);
    qt[g * D + j] = Stor<DT>::round(xo);
    qt[g * D + j + H2] = Stor<DT>::round(yo);
  }
}

template <int DT, int D, int G>
__device__ __forceinline__ void load_query(const void* q, int64_t qi, int Hq, int j, float* qs) {
  using T = typename Stor<DT>::T;
  const T* src = static_cast<const T*>(q) + (qi * Hq + static_cast<int64_t>(j) * G) * D;
  for (int i = threadIdx.x; i < G * D; i += kBlock) qs[i] = Stor<DT>::load(src + i);
}

// Indices of the (query, KV head) a workgroup serves: grid = (x, Hkv, B*T).
struct QueryCtx {
  int64_t qi;        // query index b*T + tq
  int64_t slot;      // qi*Hkv + j (selection / workspace slot)
  int64_t seq_head;  // b*Hkv + j (tree head)
  int64_t t;         // token position of the query
  const int32_t* sel;   // [n_sel][k]
  const int32_t* cnt;   // [n_sel]
};

__device__ __forceinline__ QueryCtx query_ctx(const recsa_tree& tr, int T, const int64_t* pos,
                                              const int32_t* sel, const int32_t* cnt,
                                              int n_sel) {
  QueryCtx qc;
  qc.qi = blockIdx.z;
  qc.slot = qc.qi * tr.Hkv + blockIdx.y;
  qc.seq_head = (qc.qi / T) * tr.Hkv + blockIdx.y;
  qc.t = pos[qc.qi];
  qc.sel = sel + qc.slot * n_sel * tr.k;
  qc.cnt = cnt + qc.slot * n_sel;
  return qc;
}

// ------------------------------------------------------------------ score
template <int DT, int D, int G>
__global__ void __launch_bounds__(kBlock)
    score_kernel(recsa_tree tr, const void* q, int Hq, int T, const int64_t* pos,
                 const int32_t* sel, const int32_t* cnt, float* ws_logits, int level, int n_sel,
                 int CK) {
  using T_ = typename Stor<DT>::T;
  __shared__ float qs[G * D];
  __shared__ float qt[4][G * D];
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel);
  const ListView lv = list_view(qc.t, level, tr.n_levels - 1, tr.k, qc.sel, qc.cnt);
  if (lv.len <= tr.k) return;                       // fully selected level
  const int n_others = lv.len - 1;
  const int pbase = blockIdx.x * kChunk;
  if (pbase >= n_others) return;
  load_query<DT, D, G>(q, qc.qi, Hq, blockIdx.y, qs);
  __syncthreads();
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const int p_q = lv.len - 1, r_q = p_q / kC, c_q = p_q % kC;
  const int64_t rows_l = level_rows_dev(tr.L_cap, level);
  float* out = ws_logits + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>(G) * CK;
#pragma unroll 1
  for (int gi = 0; gi < 4; ++gi) {
    const int p0 = pbase + (wid * 4 + gi) * kC;    // first position of this group
    const bool active = p0 < n_others;
    if (active) rotate_query<DT, D, G>(qs, qt[wid], kC * (r_q - p0 / kC) + c_q, tr.rope);
    __syncthreads();
    if (active) {
      const int nvalid = min(kC, n_others - p0);
      const T_* rows = static_cast<const T_*>(tr.K[level]) + (qc.seq_head * rows_l + lv.node(p0)) * D;
      float lg[G];
      group_logits<DT, D, G>(rows, nvalid, qt[wid], tr.rope, lg);
      const int c = lane >> 2, s = lane & 3;
      if (c < nvalid) {
#pragma unroll
        for (int g = 0; g < G; ++g)
          if ((g & 3) == s) out[static_cast<int64_t>(g) * CK + p0 + c] = lg[g];
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------- topk
// One workgroup per (query, KV head).  Thread i owns list positions
// [16 i, 16 i + 16) (C*k <= 4096 positions).
template <int G>
__global__ void __launch_bounds__(kBlock)
    topk_kernel(recsa_tree tr, int T, const int64_t* pos, int32_t* sel, int32_t* cnt, float* imp,
                const float* ws_logits, uint32_t* ws_bitmap, int level, int n_sel, int CK) {
  constexpr int PPT = kMaxCK / kBlock;   // 16 positions per thread
  __shared__ float red_f[kMaxG][4];
  __shared__ int red_i[4];
  __shared__ int hist[256];
  __shared__ int s_digit, s_need;
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel);
  const int k = tr.k;
  const ListView lv = list_view(qc.t, level, tr.n_levels - 1, k, qc.sel, qc.cnt);
  int32_t* out_sel = const_cast<int32_t*>(qc.sel) + static_cast<int64_t>(level - 1) * k;
  int32_t* out_cnt = const_cast<int32_t*>(qc.cnt) + (level - 1);
  float* imp_out = imp ? imp + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>(CK) : nullptr;
  uint32_t* bm = ws_bitmap + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>((CK + 31) / 32);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid >> 6;

  if (lv.len <= k) {                  // every candidate is selected
    for (int p = tid; p < k; p += kBlock)
      out_sel[p] = p < lv.len ? static_cast<int32_t>(lv.node(p)) : -1;
    if (tid == 0) *out_cnt = lv.len;
    if (imp_out)
      for (int p = tid; p < CK; p += kBlock) imp_out[p] = 0.f;
    return;
  }
  const int n = lv.len - 1;           // non-current candidates
  const float* lgs = ws_logits + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>(G) * CK;
  const int p0 = tid * PPT;

  // importance I_p = (1/G) sum_g softmax_p(s_g)
  float I[PPT];
  {
    float mx[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < PPT; ++i)
        if (p0 + i < n) m = fmaxf(m, lgs[g * CK + p0 + i]);
      m = wave_max(m);
      if (lane == 0) red_f[g][wid] = m;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g)
      mx[g] = fmaxf(fmaxf(red_f[g][0], red_f[g][1]), fmaxf(red_f[g][2], red_f[g][3]));
    __syncthreads();
    float e[G][PPT];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        e[g][i] = (p0 + i < n) ? __expf(lgs[g * CK + p0 + i] - mx[g]) : 0.f;
        sum += e[g][i];
      }
      sum = wave_sum(sum);
      if (lane == 0) red_f[g][wid] = sum;
    }
    __syncthreads();
    float invz[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
      invz[g] = 1.0f / (red_f[g][0] + red_f[g][1] + red_f[g][2] + red_f[g][3]);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      float s = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) s += e[g][i] * invz[g];
      I[i] = s * (1.0f / G);
    }
  }
  uint32_t key[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) key[i] = __float_as_uint(I[i]);   // I >= 0: order-preserving
  if (imp_out) {
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (p0 + i < CK) imp_out[p0 + i] = (p0 + i < n) ? I[i] : 0.f;
  }

  // radix select of the (k-1)-th largest key, 8 bits per pass
  uint32_t prefix = 0xFFFFFFFFu, pmask = 0;
  int need = k - 1;
  if (need > 0) prefix = 0;          // k == 1: nothing beside the current node
#pragma unroll 1
  for (int pass = 0; pass < (need > 0 ? 4 : 0); ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (p0 + i < n && (key[i] & pmask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255], 1);
    __syncthreads();
    if (wid == 0) {
      int h[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) h[b] = hist[4 * lane + b];
      const int local = h[0] + h[1] + h[2] + h[3];
      // suffix sum over lanes >= lane
      int suf = local;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        int u = __shfl_down(suf, o, kWave);
        if (lane + o < kWave) suf += u;
      }
      int above = suf - local;       // keys in bins >= 4*lane + 4
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        if (above < need && need <= above + h[b]) {
          s_digit = 4 * lane + b;
          s_need = need - above;
        }
        above += h[b];
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(s_digit) << shift;
    pmask |= 0xFFu << shift;
    need = s_need;
    __syncthreads();
  }
  // keys > prefix are in; keys == prefix are in for the first `need` positions
  int n_eq = 0;
#pragma unroll
  for (int i = 0; i < PPT; ++i) n_eq += (p0 + i < n && key[i] == prefix) ? 1 : 0;
  int tot;
  int eq_rank = block_excl_scan(n_eq, red_i, &tot);
  bool take[PPT];
  int n_take = 0;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const bool valid = p0 + i < n;
    const bool eq = valid && key[i] == prefix;
    take[i] = need > 0 && valid && (key[i] > prefix || (eq && eq_rank < need));
    eq_rank += eq ? 1 : 0;
    n_take += take[i] ? 1 : 0;
  }
  int slot = block_excl_scan(n_take, red_i, &tot);
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    if (take[i]) {
      out_sel[slot++] = static_cast<int32_t>(lv.node(p0 + i));
      bits |= 1u << ((p0 + i) & 31);
    }
  }
  // two threads share one 32-bit word
  const uint32_t other = __shfl_xor(bits, 1, kWave);
  if ((tid & 1) == 0 && p0 < CK) bm[p0 / 32] = bits | other;
  if (tid == 0) {
    out_sel[k - 1] = static_cast<int32_t>(lv.cur);
    *out_cnt = k;
  }
}

// ------------------------------------------------------------- attention
// Virtual entry space of one (query, KV head): level 0 .. n_sel-1 blocks of
// CPL*256 list positions.  Split `blockIdx.x` of n_split covers a contiguous
// range of 256-position chunks.  Level 0: every position < |A0| is an exact
// token (logit computed here).  Level l >= 1 (scored): positions < |A|-1 that
// are not selected are summaries (logit from the workspace).
template <int DT, int D, int G>
__global__ void __launch_bounds__(kBlock)
    attn_kernel(recsa_tree tr, const void* q, int Hq, int T, const int64_t* pos,
                const int32_t* sel, const int32_t* cnt, float* out, const float* ws_logits,
                const uint32_t* ws_bitmap, float* part, int n_split, int n_sel, int CK) {
  using T_ = typename Stor<DT>::T;
  constexpr int DPL = D / kWave;
  __shared__ float qs[G * D];
  __shared__ float qt[4][G * D];
  __shared__ float lg[G][kChunk];
  __shared__ float red_f[kMaxG][4];
  __shared__ float accs[4][G][D];
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid >> 6;
  const int cpl = (CK + kChunk - 1) / kChunk;          // chunks per level
  const int n_chunks = n_sel * cpl;
  const int per = n_chunks / n_split;
  const int ch_lo = blockIdx.x * per, ch_hi = ch_lo + per;
  const int top = tr.n_levels - 1;

  load_query<DT, D, G>(q, qc.qi, Hq, blockIdx.y, qs);
  __syncthreads();

  float m_run[G], l_run[G], acc[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int u = 0; u < DPL; ++u) acc[g][u] = 0.f;
  }

#pragma unroll 1
  for (int ch = ch_lo; ch < ch_hi; ++ch) {
    const int level = ch / cpl;
    const int pbase = (ch % cpl) * kChunk;
    const ListView lv = list_view(qc.t, level, top, tr.k, qc.sel, qc.cnt);
    int n_pos;                                           // candidate positions in play
    if (level == 0) {
      n_pos = lv.len;
    } else {
      if (lv.len <= tr.k) continue;                      // no summaries at this level
      n_pos = lv.len - 1;
    }
    if (pbase >= n_pos) continue;
    const int64_t rows_l = level_rows_dev(tr.L_cap, level);
    // ---- logits of the chunk into lg[g][*]
    if (level == 0) {
      const int p_q = lv.len - 1, r_q = p_q / kC, c_q = p_q % kC;
#pragma unroll 1
      for (int gi = 0; gi < 4; ++gi) {
        const int off = (wid * 4 + gi) * kC;
        const int p0 = pbase + off;
        const bool active = p0 < n_pos;
        if (active) rotate_query<DT, D, G>(qs, qt[wid], kC * (r_q - p0 / kC) + c_q, tr.rope);
        __syncthreads();
        float l[G];
        const int nvalid = active ? min(kC, n_pos - p0) : 0;
        if (active) {
          const T_* rows = static_cast<const T_*>(tr.K[0]) + (qc.seq_head * rows_l + lv.node(p0)) * D;
          group_logits<DT, D, G>(rows, nvalid, qt[wid], tr.rope, l);
        }
        const int c = lane >> 2, s = lane & 3;
        if (s == 0) {
#pragma unroll
          for (int g = 0; g < G; ++g) lg[g][off + c] = (c < nvalid) ? l[g] : -INFINITY;
        }
        __syncthreads();
      }
    } else {
      const float* src = ws_logits + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>(G) * CK;
      const uint32_t* bm = ws_bitmap + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>((CK + 31) / 32);
      const int p = pbase + tid;
      const bool ent = p < n_pos && !((bm[p >> 5] >> (p & 31)) & 1u);
#pragma unroll
      for (int g = 0; g < G; ++g) lg[g][tid] = ent ? src[static_cast<int64_t>(g) * CK + p] : -INFINITY;
      __syncthreads();
    }
    // ---- chunk max and rescale
    float mnew[G], scale_old[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = wave_max(lg[g][tid]);
      if (lane == 0) red_f[g][wid] = m;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mc = fmaxf(fmaxf(red_f[g][0], red_f[g][1]), fmaxf(red_f[g][2], red_f[g][3]));
      mnew[g] = fmaxf(m_run[g], mc);
      scale_old[g] = (m_run[g] == -INFINITY) ? 0.f : __expf(m_run[g] - mnew[g]);
    }
    __syncthreads();
    // ---- probabilities (in place) and their sum
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float v = lg[g][tid];
      const float pr = (v == -INFINITY) ? 0.f : __expf(v - mnew[g]);
      lg[g][tid] = pr;
      const float sm = wave_sum(pr);
      if (lane == 0) red_f[g][wid] = sm;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l_run[g] = l_run[g] * scale_old[g] + red_f[g][0] + red_f[g][1] + red_f[g][2] + red_f[g][3];
      m_run[g] = mnew[g];
#pragma unroll
      for (int u = 0; u < DPL; ++u) acc[g][u] *= scale_old[g];
    }
    // ---- P V over this wave's 64 positions (one row per position, lanes = dims)
    const T_* vbase = static_cast<const T_*>(tr.V[level]) + qc.seq_head * rows_l * D;
    const int lim = min(kWave, n_pos - (pbase + wid * kWave));
#pragma unroll 1
    for (int i = 0; i < lim; ++i) {
      const int pp = wid * kWave + i;
      float pw[G];
      bool any = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        pw[g] = lg[g][pp];
        any |= pw[g] != 0.f;
      }
      if (!any) continue;
      const T_* vr = vbase + lv.node(pbase + pp) * D + lane * DPL;
      float v[DPL];
      if constexpr (DPL == 2) {
        load_vec<DT, 2>(vr, v);
      } else {
        v[0] = Stor<DT>::load(vr);
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < DPL; ++u) acc[g][u] += pw[g] * v[u];
    }
    __syncthreads();
  }

  // ---- combine the four waves' partial sums
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int u = 0; u < DPL; ++u) accs[wid][g][lane * DPL + u] = acc[g][u];
  __syncthreads();
  if (n_split == 1) {
    float* o = out + (qc.qi * Hq + static_cast<int64_t>(blockIdx.y) * G) * D;
    for (int i = tid; i < G * D; i += kBlock) {
      const int g = i / D, dd = i % D;
      const float a = accs[0][g][dd] + accs[1][g][dd] + accs[2][g][dd] + accs[3][g][dd];
      o[i] = a / l_run[g];
    }
  } else {
    float* pp = part + ((qc.slot * n_split) + blockIdx.x) * static_cast<int64_t>(G) * (D + 2);
    for (int i = tid; i < G * D; i += kBlock) {
      const int g = i / D, dd = i % D;
      pp[g * (D + 2) + 2 + dd] = accs[0][g][dd] + accs[1][g][dd] + accs[2][g][dd] + accs[3][g][dd];
    }
    if (tid < G) {
      pp[tid * (D + 2)] = m_run[tid];
      pp[tid * (D + 2) + 1] = l_run[tid];
    }
  }
}

// Merge the n_split partial softmax states of each (query, head).
template <int D, int G>
__global__ void __launch_bounds__(D) combine_kernel(const float* part, float* out, int Hkv, int Hq,
                                                    int n_split) {
  const int64_t qi = blockIdx.y;
  const int j = blockIdx.x / G, g = blockIdx.x % G;
  const int64_t slot = qi * Hkv + j;
  const float* pp = part + slot * n_split * static_cast<int64_t>(G) * (D + 2) + g * (D + 2);
  const int stride = G * (D + 2);
  float m = -INFINITY;
  for (int s = 0; s < n_split; ++s) m = fmaxf(m, pp[s * stride]);
  float l = 0.f, a = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float ms = pp[s * stride];
    if (ms == -INFINITY) continue;
    const float w = __expf(ms - m);
    l += w * pp[s * stride + 1];
    a += w * pp[s * stride + 2 + threadIdx.x];
  }
  out[(qi * Hq + static_cast<int64_t>(j) * G + g) * D + threadIdx.x] = a / l;
}

// ------------------------------------------------------------- launchers
template <int DT, int D, int G>
static hipError_t select_impl(const recsa_tree& tr, const void* q, int Hq, int T,
                              const int64_t* pos, int32_t* sel, int32_t* cnt, float* imp,
                              void* ws, const WsLayout& w, hipStream_t s) {
  float* logits = reinterpret_cast<float*>(static_cast<char*>(ws) + w.logits_off);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + w.bitmap_off);
  const unsigned nq = static_cast<unsigned>(static_cast<int64_t>(tr.B) * T);
  const int cpl = (w.CK + kChunk - 1) / kChunk;
  for (int l = tr.n_levels - 1; l >= 1; --l) {
    if (l < tr.n_levels - 1) {   // the top list has at most k nodes: nothing to score
      score_kernel<DT, D, G><<<dim3(cpl, tr.Hkv, nq), kBlock, 0, s>>>(
          tr, q, Hq, T, pos, sel, cnt, logits, l, w.n_sel, w.CK);
    }
    topk_kernel<G><<<dim3(1, tr.Hkv, nq), kBlock, 0, s>>>(tr, T, pos, sel, cnt, imp, logits,
                                                          bitmap, l, w.n_sel, w.CK);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int DT, int D, int G>
static hipError_t attn_impl(const recsa_tree& tr, const void* q, int Hq, int T, const int64_t* pos,
                            const int32_t* sel, const int32_t* cnt, float* out, void* ws,
                            const WsLayout& w, bool decode, hipStream_t s) {
  const float* logits = reinterpret_cast<const float*>(static_cast<char*>(ws) + w.logits_off);
  const uint32_t* bitmap = reinterpret_cast<const uint32_t*>(static_cast<char*>(ws) + w.bitmap_off);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + w.part_off);
  const unsigned nq = static_cast<unsigned>(static_cast<int64_t>(tr.B) * T);
  const int n_split = decode ? w.n_split : 1;
  attn_kernel<DT, D, G><<<dim3(n_split, tr.Hkv, nq), kBlock, 0, s>>>(
      tr, q, Hq, T, pos, sel, cnt, out, logits, bitmap, part, n_split, w.n_sel, w.CK);
  if (n_split > 1)
    combine_kernel<D, G><<<dim3(tr.Hkv * G, nq), D, 0, s>>>(part, out, tr.Hkv, Hq, n_split);
  return hipGetLastError();
}

#define RECSA_DISPATCH(FN, ...)                                                     \
  do {                                                                              \
    const int G = Hq / tr.Hkv;                                                      \
    if (tr.dtype == RECSA_BF16 && tr.d == 128) {                                    \
      if (G == 4) return FN<RECSA_BF16, 128, 4>(__VA_ARGS__);                       \
      if (G == 1) return FN<RECSA_BF16, 128, 1>(__VA_ARGS__);                       \
      if (G == 2) return FN<RECSA_BF16, 128, 2>(__VA_ARGS__);                       \
      if (G == 8) return FN<RECSA_BF16, 128, 8>(__VA_ARGS__);                       \
    } else if (tr.dtype == RECSA_BF16 && tr.d == 64) {                              \
      if (G == 4) return FN<RECSA_BF16, 64, 4>(__VA_ARGS__);                        \
      if (G == 1) return FN<RECSA_BF16, 64, 1>(__VA_ARGS__);                        \
      if (G == 2) return FN<RECSA_BF16, 64, 2>(__VA_ARGS__);                        \
      if (G == 8) return FN<RECSA_BF16, 64, 8>(__VA_ARGS__);                        \
    } else if (tr.dtype == RECSA_F32 && tr.d == 128) {                              \
      if (G == 4) return FN<RECSA_F32, 128, 4>(__VA_ARGS__);                        \
      if (G == 1) return FN<RECSA_F32, 128, 1>(__VA_ARGS__);                        \
      if (G == 2) return FN<RECSA_F32, 128, 2>(__VA_ARGS__);                        \
      if (G == 8) return FN<RECSA_F32, 128, 8>(__VA_ARGS__);                        \
    } else if (tr.dtype == RECSA_F32 && tr.d == 64) {                               \
      if (G == 4) return FN<RECSA_F32, 64, 4>(__VA_ARGS__);                         \
      if (G == 1) return FN<RECSA_F32, 64, 1>(__VA_ARGS__);                         \
      if (G == 2) return FN<RECSA_F32, 64, 2>(__VA_ARGS__);                         \
      if (G == 8) return FN<RECSA_F32, 64, 8>(__VA_ARGS__);                         \
    }                                                                               \
    return hipErrorInvalidValue;                                                    \
  } while (0)

hipError_t launch_select(const recsa_tree& tr, const void* q, int Hq, int T, const int64_t* pos,
                         int32_t* sel, int32_t* cnt, float* imp, void* ws, const WsLayout& w,
                         hipStream_t s) {
  RECSA_DISPATCH(select_impl, tr, q, Hq, T, pos, sel, cnt, imp, ws, w, s);
}

hipError_t launch_attn(const recsa_tree& tr, const void* q, int Hq, int T, const int64_t* pos,
                       const int32_t* sel, const int32_t* cnt, float* out, void* ws,
                       const WsLayout& w, bool decode, hipStream_t s) {
  RECSA_DISPATCH(attn_impl, tr, q, Hq, T, pos, sel, cnt, out, ws, w, decode, s);
}

}  // namespace recsa
