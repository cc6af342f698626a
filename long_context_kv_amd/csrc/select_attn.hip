// Hierarchical selection (picx.dev Hierarchical Selection, Eq. 3) and the
// unified softmax (Unified Softmax, Eq. 4) with candidate-local RoPE (Key
// Theoretical Insight), split so that keys turn by their in-group offset and
// queries by the group distance ("slot-based rotation splitting", Conclusion).
//
// These are the kernels behind recsa_select / recsa_attn_decode /
// recsa_attn_prefill (any number of queries T):
//   score_kernel   -- logits of the non-current candidates of A^(l), 64 list
//                     positions (one 16-row group per wave) per workgroup;
//   topk_kernel    -- importance and exact top-(k-1) per (query, KV head);
//   attn_kernel    -- exact tokens plus unselected summaries with an online
//                     softmax, the entry groups of a query split over
//                     n_split workgroups;
//   combine_kernel -- merges the n_split partial softmax states.
// recsa_decode runs the same steps for one query per sequence in a single
// persistent launch (decode_fused.hip).
#include "recsa_common.hpp"
#include "recsa_device.hpp"
#include "recsa_kernels.hpp"

namespace recsa {

// Indices of the (query, KV head) a workgroup serves: grid = (x, Hkv, B*T).
struct QueryCtx {
  int64_t qi;        // query index b*T + tq
  int64_t slot;      // qi*Hkv + j (selection / workspace slot)
  int64_t seq_head;  // b*Hkv + j (tree head)
  int64_t t;         // token position of the query
  int32_t* sel;      // [n_sel][k]
  int32_t* cnt;      // [n_sel]
};

__device__ __forceinline__ QueryCtx query_ctx(const recsa_tree& tr, int T, const int64_t* pos,
                                              int32_t* sel, int32_t* cnt, int n_sel) {
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
    score_kernel(recsa_tree tr, const void* q, int Hq, int T, const int64_t* pos, int32_t* sel,
                 int32_t* cnt, float* ws_logits, int level, int n_sel, int CK) {
  using T_ = typename Stor<DT>::T;
  __shared__ float qs[G * D];
  __shared__ float qt[4][G * D];
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel);
  const ListView lv = list_view(qc.t, level, tr.n_levels - 1, tr.k, qc.sel, qc.cnt);
  if (lv.len <= tr.k) return;                       // fully selected level
  const int n_others = lv.len - 1;
  const int pbase = blockIdx.x * (4 * kC);
  if (pbase >= n_others) return;
  load_query_rows<DT, D, G, kBlock>(q, qc.qi * Hq + static_cast<int64_t>(blockIdx.y) * G, qs);
  __syncthreads();
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const int p0 = pbase + wid * kC;                  // this wave's group
  if (p0 >= n_others) return;                        // no block barrier below
  const int p_q = lv.len - 1;
  const int nvalid = min(kC, n_others - p0);
  const int64_t rows_l = level_rows_dev(tr.L_cap, level);
  const T_* rows = static_cast<const T_*>(tr.Kr[level]) + (qc.seq_head * rows_l + lv.node(p0)) * D;
  KRows<DT, D> kr;                       // key rows in flight during the rotation
  group_load_k<DT, D>(rows, 0, nvalid, kr);
  rotate_query<DT, D, G>(qs, qt[wid], kC * (p_q / kC - p0 / kC) + p_q % kC, tr.rope);
  wave_sync();
  float lg[G];
  group_logits_from<DT, D, G>(kr, 0, nvalid, qt[wid], tr.rope, lg);
  float* out = ws_logits + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>(G) * CK;
  const int c = lane >> 2, s = lane & 3;
  if (c < nvalid) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      if ((g & 3) == s) out[static_cast<int64_t>(g) * CK + p0 + c] = lg[g];
  }
}

// ------------------------------------------------------------------- topk
template <int G>
__global__ void __launch_bounds__(kBlock)
    topk_kernel(recsa_tree tr, int T, const int64_t* pos, int32_t* sel, int32_t* cnt, float* imp,
                const float* ws_logits, uint32_t* ws_bitmap, int level, int n_sel, int CK) {
  __shared__ TopkSmem sm;
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel);
  const int k = tr.k;
  const int top = tr.n_levels - 1;
  float* imp_q = imp ? imp + qc.slot * n_sel * static_cast<int64_t>(CK) : nullptr;
  if (level == top - 1) {             // the top list [0 .. a_top] is fully selected
    const ListView lt = list_view(qc.t, top, top, k, qc.sel, qc.cnt);
    wg_take_all<kBlock>(lt, k, qc.sel + static_cast<int64_t>(top - 1) * k, qc.cnt + (top - 1),
                        imp_q ? imp_q + static_cast<int64_t>(top - 1) * CK : nullptr, CK);
  }
  const ListView lv = list_view(qc.t, level, top, k, qc.sel, qc.cnt);
  int32_t* out_sel = qc.sel + static_cast<int64_t>(level - 1) * k;
  int32_t* out_cnt = qc.cnt + (level - 1);
  float* imp_l = imp_q ? imp_q + static_cast<int64_t>(level - 1) * CK : nullptr;
  if (lv.len <= k) {
    wg_take_all<kBlock>(lv, k, out_sel, out_cnt, imp_l, CK);
    return;
  }
  const float* lgs = ws_logits + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>(G) * CK;
  uint32_t* bm = ws_bitmap + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>((CK + 31) / 32);
  wg_topk<G, kBlock>(lgs, lv.len - 1, k, CK, lv, out_sel, out_cnt, bm, imp_l, sm);
}

// ------------------------------------------------------------- attention
// Entry groups of one (query, KV head) dealt round-robin to n_split workgroups.
template <int DT, int D, int G>
__global__ void __launch_bounds__(kBlock)
    attn_kernel(recsa_tree tr, const void* q, int Hq, int T, const int64_t* pos, int32_t* sel,
                int32_t* cnt, float* out, const float* ws_logits, const uint32_t* ws_bitmap,
                float* part, int n_split, int n_sel, int CK) {
  __shared__ float qs[G * D];
  __shared__ AttnSmem<D, G, kBlock> sm;
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel);
  load_query_rows<DT, D, G, kBlock>(q, qc.qi * Hq + static_cast<int64_t>(blockIdx.y) * G, qs);
  __syncthreads();
  const EntryGroups eg = entry_groups(qc.t, tr, n_sel, qc.sel, qc.cnt);
  const float* lg_slot = ws_logits + qc.slot * n_sel * static_cast<int64_t>(G) * CK;
  const uint32_t* bm_slot = ws_bitmap + qc.slot * n_sel * static_cast<int64_t>((CK + 31) / 32);
  attn_groups<DT, D, G, kBlock>(tr, qc.t, qc.seq_head, qc.sel, qc.cnt, eg, blockIdx.x, n_split, qs,
                                lg_slot, bm_slot, CK, nullptr, nullptr, sm);
  if (n_split == 1) {
    float* o = out + (qc.qi * Hq + static_cast<int64_t>(blockIdx.y) * G) * D;
    for (int e = threadIdx.x; e < G * D; e += kBlock) o[e] = sm.wacc[0][e / D][e % D] / sm.res_l[e / D];
  } else {
    float* pp = part + ((qc.slot * n_split) + blockIdx.x) * static_cast<int64_t>(G) * (D + 2);
    for (int e = threadIdx.x; e < G * D; e += kBlock)
      pp[(e / D) * (D + 2) + 2 + e % D] = sm.wacc[0][e / D][e % D];
    if (threadIdx.x < G) {
      pp[threadIdx.x * (D + 2)] = sm.res_m[threadIdx.x];
      pp[threadIdx.x * (D + 2) + 1] = sm.res_l[threadIdx.x];
    }
  }
}

template <int D, int G>
__global__ void __launch_bounds__(kBlock) combine_kernel(const float* part, float* out, int Hkv,
                                                         int Hq, int n_split) {
  const int64_t qi = blockIdx.y;
  const int j = blockIdx.x;
  const float* pp = part + (qi * Hkv + j) * n_split * static_cast<int64_t>(G) * (D + 2);
  merge_partials<D, G, kBlock>(pp, n_split, out + (qi * Hq + static_cast<int64_t>(j) * G) * D);
}

// ------------------------------------------------------------- launchers
template <int DT, int D, int G>
static hipError_t select_impl(const recsa_tree& tr, const void* q, int Hq, int T,
                              const int64_t* pos, int32_t* sel, int32_t* cnt, float* imp,
                              void* ws, const WsLayout& w, hipStream_t s) {
  float* logits = reinterpret_cast<float*>(static_cast<char*>(ws) + w.logits_off);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + w.bitmap_off);
  const unsigned nq = static_cast<unsigned>(static_cast<int64_t>(tr.B) * T);
  const int top = tr.n_levels - 1;
  const unsigned score_blocks = static_cast<unsigned>((w.CK + 4 * kC - 1) / (4 * kC));
  // the top list never needs scoring; the top-k of level top-1 also writes
  // the top level's (full) selection
  const int first = top >= 2 ? top - 1 : top;
  for (int l = first; l >= 1; --l) {
    if (l < top)
      score_kernel<DT, D, G><<<dim3(score_blocks, tr.Hkv, nq), kBlock, 0, s>>>(
          tr, q, Hq, T, pos, sel, cnt, logits, l, w.n_sel, w.CK);
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
      tr, q, Hq, T, pos, const_cast<int32_t*>(sel), const_cast<int32_t*>(cnt), out, logits, bitmap,
      part, n_split, w.n_sel, w.CK);
  if (n_split > 1)
    combine_kernel<D, G><<<dim3(tr.Hkv, nq), kBlock, 0, s>>>(part, out, tr.Hkv, Hq, n_split);
  return hipGetLastError();
}

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
