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
#include <algorithm>

#include "recsa_common.hpp"
#include "recsa_device.hpp"
#include "recsa_kernels.hpp"
#include "recsa_mfma.hpp"

namespace recsa {

// Indices of the (query, KV head) a workgroup serves: grid = (n_x*B*T, Hkv),
// blockIdx.x = qi*n_x + x.  The KV head is the slowest launch dimension, so
// the workgroups in flight at any time read one head's rows (one head's
// level 0 is a few hundred MB, about the size of the last-level cache;
// every head at once is not).
struct QueryCtx {
  int64_t qi;        // query index b*T + tq
  int j;             // KV head
  int x;             // index along the per-query launch dimension
  int64_t slot;      // qi*Hkv + j (selection / workspace slot)
  int64_t seq_head;  // b*Hkv + j (tree head)
  int64_t t;         // token position of the query
  int32_t* sel;      // [n_sel][k]
  int32_t* cnt;      // [n_sel]
};

__device__ __forceinline__ QueryCtx query_ctx(const recsa_tree& tr, int T, const int64_t* pos,
                                              int32_t* sel, int32_t* cnt, int n_sel, int n_x) {
  QueryCtx qc;
  qc.qi = blockIdx.x / n_x;
  qc.x = static_cast<int>(blockIdx.x % n_x);
  qc.j = static_cast<int>(blockIdx.y);
  qc.slot = qc.qi * tr.Hkv + qc.j;
  qc.seq_head = (qc.qi / T) * tr.Hkv + qc.j;
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
  __shared__ __align__(16) float qt[4][G * D];
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel, (CK + 4 * kC - 1) / (4 * kC));
  const ListView lv = list_view(qc.t, level, tr.n_levels - 1, tr.k, qc.sel, qc.cnt);
  if (lv.len <= tr.k) return;                       // fully selected level
  const int n_others = lv.len - 1;
  const int pbase = qc.x * (4 * kC);
  if (pbase >= n_others) return;
  load_query_rows<DT, D, G, kBlock>(q, qc.qi * Hq + static_cast<int64_t>(qc.j) * G, qs);
  __syncthreads();
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const int p0 = pbase + wid * kC;                  // this wave's group
  if (p0 >= n_others) return;                        // no block barrier below
  const int p_q = lv.len - 1;
  const int nvalid = min(kC, n_others - p0);
  const int64_t rows_l = level_rows_dev(tr.L_cap, level);
  const T_* rows = static_cast<const T_*>(tr.Kr[level]) + (qc.seq_head * rows_l + lv.node(p0)) * D;
  const int phi = p_q - p0;                 // = C (r_q - r) + c_q, r = p0 / C
  float* out = ws_logits + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>(G) * CK;
  if constexpr (DT == RECSA_BF16) {
    MFrag<D> kf, qf;                       // key rows in flight during the rotation
    load_key_frag<D>(rows, nvalid, kf);
    rotate_query<DT, D, G>(qs, qt[wid], phi, tr.rope);
    wave_sync();
    query_frag_lds<D, G>(reinterpret_cast<const uint16_t*>(qt[wid]), qf);
    const f32x4_t c = mfma_logits<D>(qf, kf);
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    if (lane < nvalid && lane < kC) {
#pragma unroll
      for (int g = 0; g < G; ++g) out[static_cast<int64_t>(g) * CK + p0 + lane] = c[g] * scale;
    }
  } else {
    KRows<DT, D> kr;                       // key rows in flight during the rotation
    group_load_k<DT, D>(rows, 0, nvalid, kr);
    rotate_query<DT, D, G>(qs, qt[wid], phi, tr.rope);
    wave_sync();
    float lg[G];
    group_logits_from<DT, D, G>(kr, 0, nvalid, qt[wid], tr.rope, lg);
    const int c = lane >> 2, s = lane & 3;
    if (c < nvalid) {
#pragma unroll
      for (int g = 0; g < G; ++g)
        if ((g & 3) == s) out[static_cast<int64_t>(g) * CK + p0 + c] = lg[g];
    }
  }
}

// ------------------------------------------------------------------- topk
template <int G>
__global__ void __launch_bounds__(kBlock)
    topk_kernel(recsa_tree tr, int T, const int64_t* pos, int32_t* sel, int32_t* cnt, float* imp,
                const float* ws_logits, uint32_t* ws_bitmap, int level, int n_sel, int CK) {
  __shared__ TopkSmem sm;
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel, 1);
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
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel, n_split);
  load_query_rows<DT, D, G, kBlock>(q, qc.qi * Hq + static_cast<int64_t>(qc.j) * G, qs);
  __syncthreads();
  const EntryGroups eg = entry_groups(qc.t, tr, n_sel, qc.sel, qc.cnt);
  const float* lg_slot = ws_logits + qc.slot * n_sel * static_cast<int64_t>(G) * CK;
  const uint32_t* bm_slot = ws_bitmap + qc.slot * n_sel * static_cast<int64_t>((CK + 31) / 32);
  attn_groups<DT, D, G, kBlock>(tr, qc.t, qc.seq_head, qc.sel, qc.cnt, eg, qc.x, n_split, qs,
                                lg_slot, bm_slot, CK, nullptr, nullptr, sm);
  if (n_split == 1) {
    float* o = out + (qc.qi * Hq + static_cast<int64_t>(qc.j) * G) * D;
    for (int e = threadIdx.x; e < G * D; e += kBlock) o[e] = sm.wacc[0][e / D][e % D] / sm.res_l[e / D];
  } else {
    float* pp = part + ((qc.slot * n_split) + qc.x) * static_cast<int64_t>(G) * (D + 2);
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

// ------------------------------------------------------ bucketed scoring
// Many queries per call (prefill chunks).  The list of a query at level l is
// the children of its parents -- S^(l+1), or the whole prefix when level l+1
// is fully selected -- C rows per parent in parent order, so list group r of
// query q holds the C rows under its r-th parent u.  Each (query, group)
// pair is filed under the bucket (sequence, KV head, u); a wave loads the
// parent's C rotated key rows once, as the B operand, and scores them
// against C/G of the bucket's queries per matrix instruction, each query
// row rotated by its own phi = p_q - C r.  The logits are the float32 values
// the per-query kernel computes (same operands, same k order).
struct BucketArgs {
  int32_t* count;       // [n_keys] entries per bucket
  int32_t* off;         // [n_keys] first entry of each bucket
  int32_t* cursor;      // [n_keys] next free entry while filing
  int32_t* tile_key;    // [max_tiles] bucket of each tile
  int32_t* tile_first;  // [max_tiles] first entry of each tile
  uint2* entries;       // [max_entries] {query index, phi | r << 12 | nvalid << 20}
  int32_t* n_tiles;     // tiles of this level
  int n_keys;           // B * Hkv * n_up
  int64_t n_up;         // parents per (sequence, KV head): N_{l+1} + 1
};

__global__ void bucket_clear_kernel(BucketArgs ba) {
  const int i0 = blockIdx.x * blockDim.x + threadIdx.x;
  for (int i = i0; i < ba.n_keys; i += gridDim.x * blockDim.x) ba.count[i] = 0;
  if (i0 == 0) *ba.n_tiles = 0;
}

// FILE = false: count the entries of every bucket; true: file them.
// Grid (n_queries, Hkv); thread r takes list group r.
template <bool FILE>
__global__ void __launch_bounds__(kBlock)
    bucket_file_kernel(recsa_tree tr, int T, const int64_t* pos, int32_t* sel, int32_t* cnt,
                       int level, int n_sel, BucketArgs ba) {
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel, 1);
  const ListView lv = list_view(qc.t, level, tr.n_levels - 1, tr.k, qc.sel, qc.cnt);
  if (lv.len <= tr.k) return;                       // fully selected level
  const int n = lv.len - 1;                         // scored positions [0, n)
  const int ng = (n + kC - 1) / kC;
  for (int r = threadIdx.x; r < ng; r += kBlock) {
    const int64_t key = qc.seq_head * ba.n_up + lv.node(r * kC) / kC;
    if constexpr (!FILE) {
      atomicAdd(&ba.count[key], 1);
    } else {
      const int at = atomicAdd(&ba.cursor[key], 1);
      const uint32_t phi = static_cast<uint32_t>(n - r * kC);      // p_q - C r
      const uint32_t nvalid = static_cast<uint32_t>(min(kC, n - r * kC));
      ba.entries[at] = make_uint2(static_cast<uint32_t>(qc.qi),
                                  phi | (static_cast<uint32_t>(r) << 12) | (nvalid << 20));
    }
  }
}

// One workgroup: bucket offsets (exclusive scan of the counts), fill
// cursors, and the tile list (every bucket cut into kBucketTile entries).
constexpr int kScanThreads = 1024;
__global__ void __launch_bounds__(kScanThreads) bucket_scan_kernel(BucketArgs ba) {
  __shared__ int red[2][kScanThreads / kWave];
  const int per = (ba.n_keys + kScanThreads - 1) / kScanThreads;
  const int k0 = min(static_cast<int>(threadIdx.x) * per, ba.n_keys);
  const int k1 = min(k0 + per, ba.n_keys);
  int ne = 0, nt = 0;
  for (int key = k0; key < k1; ++key) {
    const int c = ba.count[key];
    ne += c;
    nt += (c + kBucketTile - 1) / kBucketTile;
  }
  int tot_e, tot_t;
  int oe = block_scan_excl<kScanThreads>(ne, red[0], &tot_e);
  int ot = block_scan_excl<kScanThreads>(nt, red[1], &tot_t);
  for (int key = k0; key < k1; ++key) {
    const int c = ba.count[key];
    ba.off[key] = oe;
    ba.cursor[key] = oe;
    for (int f = 0; f < c; f += kBucketTile) {
      ba.tile_key[ot] = key;
      ba.tile_first[ot] = oe + f;
      ++ot;
    }
    oe += c;
  }
  if (threadIdx.x == 0) *ba.n_tiles = tot_t;
}

// Waves take tiles (grid-stride); per tile the parent's rows stay in
// registers while C/G entries at a time are rotated and scored.
template <int D, int G>
__global__ void __launch_bounds__(kBlock)
    bucket_score_kernel(recsa_tree tr, const void* q, int Hq, float* ws_logits, int level,
                        int n_sel, int CK, BucketArgs ba) {
  constexpr int EPM = kC / G;                       // entries per matrix instruction
  constexpr int NW = kBlock / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  const int m = lane & 15, h = lane >> 4;
  const int64_t rows_l = level_rows_dev(tr.L_cap, level);
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const int n_tiles = *ba.n_tiles;
  for (int tl = blockIdx.x * NW + wid; tl < n_tiles; tl += gridDim.x * NW) {
    const int key = ba.tile_key[tl];
    const int first = ba.tile_first[tl];
    const int end = min(first + kBucketTile, ba.off[key] + ba.count[key]);
    const int64_t sh = key / ba.n_up, u = key % ba.n_up;
    const int j = static_cast<int>(sh % tr.Hkv);
    MFrag<D> kf;
    load_key_frag<D>(static_cast<const uint16_t*>(tr.Kr[level]) + (sh * rows_l + u * kC) * D,
                     static_cast<int>(min<int64_t>(kC, rows_l - u * kC)), kf);
    for (int e0 = first; e0 < end; e0 += EPM) {
      // A row m: entry e0 + m / G, query head m % G
      const int ei = e0 + m / G;
      const bool ev = ei < end;
      const uint2 ent = ev ? ba.entries[ei] : make_uint2(0u, 0u);
      const uint16_t* qrow =
          qb + (static_cast<int64_t>(ent.x) * Hq + static_cast<int64_t>(j) * G + m % G) * D;
      MFrag<D> qf;
      rotated_query_frag<D>(qrow, static_cast<int>(ent.y & 0xFFFu), tr.rope, ev, qf);
      const f32x4_t c = mfma_logits<D>(qf, kf);
      // this lane holds rows 4h + i of column m: entry (4h + i) / G, head (4h + i) % G
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * h + i;
        const int er = row / G, g = row % G;
        const uint32_t ex = __shfl(ent.x, er * G);
        const uint32_t ey = __shfl(ent.y, er * G);
        const int r = static_cast<int>((ey >> 12) & 0xFFu);
        const int nvalid = static_cast<int>((ey >> 20) & 0x1Fu);
        if (e0 + er < end && m < nvalid) {
          const int64_t slot = static_cast<int64_t>(ex) * tr.Hkv + j;
          ws_logits[((slot * n_sel + (level - 1)) * G + g) * static_cast<int64_t>(CK) + r * kC + m] =
              c[i] * scale;
        }
      }
    }
  }
}

static BucketArgs bucket_args(const recsa_tree& tr, void* ws, const WsLayout& w, int level) {
  char* b = static_cast<char*>(ws);
  BucketArgs ba;
  ba.count = reinterpret_cast<int32_t*>(b + w.bk_count_off);
  ba.off = reinterpret_cast<int32_t*>(b + w.bk_off_off);
  ba.cursor = reinterpret_cast<int32_t*>(b + w.bk_cursor_off);
  ba.tile_key = reinterpret_cast<int32_t*>(b + w.bk_tkey_off);
  ba.tile_first = reinterpret_cast<int32_t*>(b + w.bk_tfirst_off);
  ba.entries = reinterpret_cast<uint2*>(b + w.bk_entries_off);
  ba.n_tiles = reinterpret_cast<int32_t*>(b + w.bk_ntiles_off);
  ba.n_up = level_rows_host(tr.L_cap, level + 1) + 1;     // + the incomplete current node
  ba.n_keys = static_cast<int>(static_cast<int64_t>(tr.B) * tr.Hkv * ba.n_up);
  return ba;
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
    if (l < top) {
      bool scored = false;
      if constexpr (DT == RECSA_BF16) {
        if (w.bucket) {
          const BucketArgs ba = bucket_args(tr, ws, w, l);
          const unsigned clear_blocks = static_cast<unsigned>(std::min(1024, (ba.n_keys + 255) / 256));
          bucket_clear_kernel<<<clear_blocks, 256, 0, s>>>(ba);
          bucket_file_kernel<false><<<dim3(nq, tr.Hkv), kBlock, 0, s>>>(tr, T, pos, sel, cnt, l,
                                                                        w.n_sel, ba);
          bucket_scan_kernel<<<1, kScanThreads, 0, s>>>(ba);
          bucket_file_kernel<true><<<dim3(nq, tr.Hkv), kBlock, 0, s>>>(tr, T, pos, sel, cnt, l,
                                                                       w.n_sel, ba);
          const int64_t wgs = (w.bk_max_tiles + kBlock / kWave - 1) / (kBlock / kWave);
          bucket_score_kernel<D, G><<<static_cast<unsigned>(std::min<int64_t>(wgs, 8192)), kBlock,
                                      0, s>>>(tr, q, Hq, logits, l, w.n_sel, w.CK, ba);
          scored = true;
        }
      }
      if (!scored)
        score_kernel<DT, D, G><<<dim3(score_blocks * nq, tr.Hkv), kBlock, 0, s>>>(
            tr, q, Hq, T, pos, sel, cnt, logits, l, w.n_sel, w.CK);
    }
    topk_kernel<G><<<dim3(nq, tr.Hkv), kBlock, 0, s>>>(tr, T, pos, sel, cnt, imp, logits,
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
  attn_kernel<DT, D, G><<<dim3(static_cast<unsigned>(n_split) * nq, tr.Hkv), kBlock, 0, s>>>(
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
