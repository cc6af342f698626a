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
  const bool raw = tr.Kr[level] == nullptr;        // no rotated copy: rotate the key rows here
  const T_* rows = static_cast<const T_*>(raw ? tr.K[level] : tr.Kr[level]) +
                   (qc.seq_head * rows_l + lv.node(p0)) * D;
  const int phi = p_q - p0;                 // = C (r_q - r) + c_q, r = p0 / C
  float* out = ws_logits + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>(G) * CK;
  if constexpr (DT == RECSA_BF16) {
    // the table row first (the rotation waits only for it), then the key
    // rows, in flight during the rotation
    MFrag<D> kf, qf;
    QRope<DT, D, G> rq;
    load_query_rope<DT, D, G>(phi, tr.rope, rq);
    load_key_frag<D>(rows, nvalid, kf);
    rotate_query_from<DT, D, G>(qs, qt[wid], rq);
    if (raw) rotate_key_frag<D>(kf, tr.rope);
    wave_sync();
    query_frag_lds<D, G>(reinterpret_cast<const uint16_t*>(qt[wid]), qf);
    const f32x4_t c = mfma_logits<D>(qf, kf);
    store_logit_tile<D, G>(c, out, CK, p0, nvalid);
  } else {
    KRows<DT, D> kr;                       // key rows in flight during the rotation
    QRope<DT, D, G> rq;
    load_query_rope<DT, D, G>(phi, tr.rope, rq);
    group_load_k<DT, D>(rows, 0, nvalid, kr);
    rotate_query_from<DT, D, G>(qs, qt[wid], rq);
    wave_sync();
    float lg[G];
    group_logits_any<DT, D, G>(raw, kr, 0, nvalid, qt[wid], tr.rope, lg);
    const int c = lane >> 2, s = lane & 3;
    if (c < nvalid) {
#pragma unroll
      for (int g = 0; g < G; ++g)
        if ((g & 3) == s) out[static_cast<int64_t>(g) * CK + p0 + c] = lg[g];
    }
  }
}

// ------------------------------------------------------------------- topk
// NT threads per (query, KV head); lists of up to CKM positions.
template <int G, int NT, int CKM>
__global__ void __launch_bounds__(NT)
    topk_kernel(recsa_tree tr, int T, const int64_t* pos, int32_t* sel, int32_t* cnt, float* imp,
                const float* ws_logits, uint32_t* ws_bitmap, int level, int n_sel, int CK) {
  __shared__ TopkSmem sm;
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel, 1);
  const int k = tr.k;
  const int top = tr.n_levels - 1;
  float* imp_q = imp ? imp + qc.slot * n_sel * static_cast<int64_t>(CK) : nullptr;
  if (level == top - 1) {             // the top list [0 .. a_top] is fully selected
    const ListView lt = list_view(qc.t, top, top, k, qc.sel, qc.cnt);
    wg_take_all<NT>(lt, k, qc.sel + static_cast<int64_t>(top - 1) * k, qc.cnt + (top - 1),
                        imp_q ? imp_q + static_cast<int64_t>(top - 1) * CK : nullptr, CK);
  }
  const ListView lv = list_view(qc.t, level, top, k, qc.sel, qc.cnt);
  int32_t* out_sel = qc.sel + static_cast<int64_t>(level - 1) * k;
  int32_t* out_cnt = qc.cnt + (level - 1);
  float* imp_l = imp_q ? imp_q + static_cast<int64_t>(level - 1) * CK : nullptr;
  if (lv.len <= k) {
    wg_take_all<NT>(lv, k, out_sel, out_cnt, imp_l, CK);
    return;
  }
  const float* lgs = ws_logits + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>(G) * CK;
  uint32_t* bm = ws_bitmap + (qc.slot * n_sel + (level - 1)) * static_cast<int64_t>((CK + 31) / 32);
  wg_topk<G, NT, CKM>(lgs, lv.len - 1, k, CK, lv, out_sel, out_cnt, bm, imp_l, sm);
}

// ------------------------------------------------------------- attention
// Entry groups of one (query, KV head) dealt round-robin to n_split workgroups.
// SPLIT (decode calls, a few queries over many workgroups): two-group
// level-0 chunks with matrix-core logits and four-group summary chunks, the
// shape of the fused decode.  Without it (prefill, many queries): chunks of
// four groups in list order, logits on the vector units -- the faster form
// when every CU holds many such workgroups.
template <int DT, int D, int G, bool SPLIT>
__global__ void __launch_bounds__(kBlock)
    attn_kernel(recsa_tree tr, const void* q, int Hq, int T, const int64_t* pos, int32_t* sel,
                int32_t* cnt, float* out, const float* ws_logits, const uint32_t* ws_bitmap,
                float* part, int n_split, int n_sel, int CK) {
  __shared__ float qs[G * D];
  __shared__ AttnSmem<D, G, kBlock> sm;
  // this query's selections S^(l) [n_sel][k] and counts [n_sel], staged in
  // LDS once: every chunk maps its entries to nodes through them, and from
  // global memory that would be two dependent round trips per chunk
  extern __shared__ int32_t s_dyn[];
  const QueryCtx qc = query_ctx(tr, T, pos, sel, cnt, n_sel, n_split);
  int32_t* s_sel = s_dyn;
  int32_t* s_cnt = s_dyn + n_sel * tr.k;
  for (int i = threadIdx.x; i < n_sel * tr.k; i += kBlock) s_sel[i] = qc.sel[i];
  if (threadIdx.x < n_sel) s_cnt[threadIdx.x] = qc.cnt[threadIdx.x];
  load_query_rows<DT, D, G, kBlock>(q, qc.qi * Hq + static_cast<int64_t>(qc.j) * G, qs);
  __syncthreads();
  const EntryGroups eg = entry_groups(qc.t, tr, n_sel, s_sel, s_cnt);
  const float* lg_slot = ws_logits + qc.slot * n_sel * static_cast<int64_t>(G) * CK;
  const uint32_t* bm_slot = ws_bitmap + qc.slot * n_sel * static_cast<int64_t>((CK + 31) / 32);
  attn_groups<DT, D, G, kBlock, SPLIT ? 2 : 4, SPLIT>(tr, qc.t, qc.seq_head, s_sel, s_cnt, eg,
                                                     qc.x, n_split, qs, lg_slot, bm_slot, CK,
                                                     nullptr, nullptr, sm);
  if (n_split == 1) {
    float* o = out + (qc.qi * Hq + static_cast<int64_t>(qc.j) * G) * D;
    for (int e = threadIdx.x; e < G * D; e += kBlock) o[e] = sm.wacc[0][e / D][e % D] / sm.res_l[e / D];
  } else {
    float* pp = part + ((qc.slot * n_split) + qc.x) * static_cast<int64_t>(G) * (D + kPartHead);
    for (int e = threadIdx.x; e < G * D; e += kBlock)
      pp[(e / D) * (D + kPartHead) + kPartHead + e % D] = sm.wacc[0][e / D][e % D];
    if (threadIdx.x < G) {
      pp[threadIdx.x * (D + kPartHead)] = sm.res_m[threadIdx.x];
      pp[threadIdx.x * (D + kPartHead) + 1] = sm.res_l[threadIdx.x];
    }
  }
}

template <int D, int G>
__global__ void __launch_bounds__(kBlock) combine_kernel(const float* part, float* out, int Hkv,
                                                         int Hq, int n_split) {
  const int64_t qi = blockIdx.y;
  const int j = blockIdx.x;
  const float* pp = part + (qi * Hkv + j) * n_split * static_cast<int64_t>(G) * (D + kPartHead);
  merge_partials<D, G, kBlock>(pp, n_split, out + (qi * Hq + static_cast<int64_t>(j) * G) * D);
}

// ------------------------------------------------------ bucketed scoring
// Many queries per call (prefill chunks).  The list of a query at level l is
// the children of its parents -- S^(l+1), or the whole prefix when level l+1
// is fully selected -- C rows per parent in parent order, so list group r of
// query q holds the C rows under its r-th parent u.  A filing workgroup
// takes kFileQueries queries of one sequence and one KV head and sorts
// their (query, group) pairs by parent into its own region of the entry
// array (an LDS histogram, its scan, then LDS ranks); each run of one
// parent becomes tiles of at most kBucketTile entries.  A scoring wave then
// loads a parent's C rotated key rows once, as the B operand, and scores them
// against C entries at a time, each query row rotated by its own
// phi = p_q - C r.  The logits are the float32 values the per-query kernel
// computes (same operands, same k order).
struct BucketArgs {
  uint4* tiles;         // [max_tiles] {first entry, entries, sequence*Hkv + head, parent}
  uint2* entries;       // [regions][kFileQueries * k] {query index, phi | r << 13 | nvalid << 22}
  int32_t* n_tiles;     // tiles of this level
  int n_up;             // parents per (sequence, KV head): N_{l+1} + 1
};

__global__ void bucket_clear_kernel(BucketArgs ba) {
  if (threadIdx.x == 0) *ba.n_tiles = 0;
}

// Grid (B * ceil(T / kFileQueries), Hkv).
__global__ void __launch_bounds__(kBlock)
    bucket_file_kernel(recsa_tree tr, int T, const int64_t* pos, const int32_t* sel,
                       const int32_t* cnt, int level, int n_sel, BucketArgs ba) {
  constexpr int NW = kBlock / kWave;
  __shared__ int bins[kFileMaxUp];          // counts, then entry offsets / ranks
  __shared__ int red[NW];
  __shared__ int s_len[kFileQueries];       // |A^(l)| of each query
  __shared__ int64_t s_up[kFileQueries];    // offset of S^(l+1) in sel, -1 for a prefix list
  __shared__ int s_tile0;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  const int k = tr.k, top = tr.n_levels - 1, n_up = ba.n_up;
  const int nblk = (T + kFileQueries - 1) / kFileQueries;
  const int b = static_cast<int>(blockIdx.x) / nblk;
  const int tq0 = (static_cast<int>(blockIdx.x) % nblk) * kFileQueries;
  const int nq = min(kFileQueries, T - tq0);
  const int j = static_cast<int>(blockIdx.y);
  const int64_t seq_head = static_cast<int64_t>(b) * tr.Hkv + j;
  const int64_t qi0 = static_cast<int64_t>(b) * T + tq0;
  const int64_t region = (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) *
                         static_cast<int64_t>(kFileQueries) * k;
  // list geometry of every query (one query per thread)
  for (int i = threadIdx.x; i < nq; i += kBlock) {
    const int64_t slot = (qi0 + i) * tr.Hkv + j;
    const ListView lv = list_view(pos[qi0 + i], level, top, k, sel + slot * n_sel * k,
                                  cnt + slot * n_sel);
    s_len[i] = lv.len;
    s_up[i] = lv.up ? (lv.up - sel) : -1;
  }
  for (int i = threadIdx.x; i < n_up; i += kBlock) bins[i] = 0;
  __syncthreads();
  // pass 1: entries per parent
  for (int i = wid; i < nq; i += NW) {
    const int len = s_len[i];
    if (len <= k) continue;                          // fully selected level
    const int ng = (len - 1 + kC - 1) / kC;
    const int32_t* up = s_up[i] >= 0 ? sel + s_up[i] : nullptr;
    for (int r = lane; r < ng; r += kWave) atomicAdd(&bins[up ? up[r] : r], 1);
  }
  __syncthreads();
  // entry offsets and tiles: thread t owns parents [t*per, (t+1)*per)
  const int per = (n_up + kBlock - 1) / kBlock;
  const int u0 = min(static_cast<int>(threadIdx.x) * per, n_up), u1 = min(u0 + per, n_up);
  int ne = 0, nt = 0;
  for (int u = u0; u < u1; ++u) {
    ne += bins[u];
    nt += (bins[u] + kBucketTile - 1) / kBucketTile;
  }
  int tot_e, tot_t;
  int oe = block_scan_excl<kBlock>(ne, red, &tot_e);
  int ot = block_scan_excl<kBlock>(nt, red, &tot_t);
  if (threadIdx.x == 0) s_tile0 = tot_t ? atomicAdd(ba.n_tiles, tot_t) : 0;
  __syncthreads();
  ot += s_tile0;
  for (int u = u0; u < u1; ++u) {
    const int c = bins[u];
    for (int f = 0; f < c; f += kBucketTile)
      ba.tiles[ot++] = make_uint4(static_cast<uint32_t>(region + oe + f),
                                  static_cast<uint32_t>(min(kBucketTile, c - f)),
                                  static_cast<uint32_t>(seq_head), static_cast<uint32_t>(u));
    bins[u] = oe;
    oe += c;
  }
  __syncthreads();
  // pass 2: file each entry at its parent's next free slot
  for (int i = wid; i < nq; i += NW) {
    const int len = s_len[i];
    if (len <= k) continue;
    const int n = len - 1;                           // scored positions [0, n)
    const int ng = (n + kC - 1) / kC;
    const int32_t* up = s_up[i] >= 0 ? sel + s_up[i] : nullptr;
    for (int r = lane; r < ng; r += kWave) {
      const int at = atomicAdd(&bins[up ? up[r] : r], 1);
      const uint32_t phi = static_cast<uint32_t>(n - r * kC);      // p_q - C r
      const uint32_t nvalid = static_cast<uint32_t>(min(kC, n - r * kC));
      ba.entries[region + at] = make_uint2(static_cast<uint32_t>(qi0 + i),
                                           phi | (static_cast<uint32_t>(r) << 13) | (nvalid << 22));
    }
  }
}

// Waves take tiles (grid-stride); per tile the parent's rows stay in
// registers.  A rows are 16 bucket entries of one query head: each lane
// loads the table row of its entry once, then rotates and scores the G
// heads in turn; the next 16 entries are fetched while these are scored.
// Rows past the tile's end compute with query 0 at phi 0 and are not stored.
template <int D, int G>
__global__ void __launch_bounds__(kBlock)
    bucket_score_kernel(recsa_tree tr, const void* q, int Hq, float* ws_logits, int level,
                        int n_sel, int CK, BucketArgs ba) {
  constexpr int NW = kBlock / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  const int m = lane & 15, h = lane >> 4;
  const int64_t rows_l = level_rows_dev(tr.L_cap, level);
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const bool raw = tr.Kr[level] == nullptr;        // no rotated copy: rotate the key rows here
  const int n_tiles = *ba.n_tiles;
  // XCD-aware order: the device deals workgroups to its 8 XCDs round-robin,
  // so XCD x = blockIdx % 8 walks the x-th eighth of the tile array in order;
  // the tiles sit region by region (256 queries of one KV head each), so an
  // XCD's concurrent tiles share few queries' rows, which its L2 keeps
  constexpr int kXcd = 8;
  const int x = static_cast<int>(blockIdx.x % kXcd);
  const int nbx = static_cast<int>(gridDim.x / kXcd);
  const int per = (n_tiles + kXcd - 1) / kXcd;
  const int t_end = min(n_tiles, (x + 1) * per);
  for (int tl = x * per + static_cast<int>(blockIdx.x / kXcd) * NW + wid; tl < t_end;
       tl += nbx * NW) {
    const uint4 tile = ba.tiles[tl];
    const int64_t first = tile.x, end = first + tile.y;
    const int64_t sh = tile.z, u = tile.w;
    const int j = static_cast<int>(sh % tr.Hkv);
    MFrag<D> kf;
    load_key_frag<D>(static_cast<const uint16_t*>(raw ? tr.K[level] : tr.Kr[level]) +
                         (sh * rows_l + u * kC) * D,
                     static_cast<int>(min<int64_t>(kC, rows_l - u * kC)), kf);
    if (raw) rotate_key_frag<D>(kf, tr.rope);
    uint2 nxt = first + m < end ? ba.entries[first + m] : make_uint2(0u, 0u);
    for (int64_t e0 = first; e0 < end; e0 += kC) {
      const uint2 ent = nxt;                         // A row m: entry e0 + m
      nxt = e0 + kC + m < end ? ba.entries[e0 + kC + m] : make_uint2(0u, 0u);
      RopeFrag<D> rf;
      load_rope_frag<D>(static_cast<int>(ent.y & 0x1FFFu), tr.rope, rf);
      // this lane's output rows 4h + i: entry e0 + 4h + i (held by lane 4h + i)
      uint32_t ox[4], oy[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ox[i] = __shfl(ent.x, 4 * h + i);
        oy[i] = __shfl(ent.y, 4 * h + i);
      }
      const uint16_t* qrow = qb + (static_cast<int64_t>(ent.x) * Hq + static_cast<int64_t>(j) * G) * D;
#pragma unroll 1
      for (int g = 0; g < G; ++g) {
        MFrag<D> qf;
        rotate_frag<D>(qrow + g * D, rf, qf);
        const f32x4_t c = mfma_logits<D>(qf, kf);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = static_cast<int>((oy[i] >> 13) & 0x1FFu);
          const int nvalid = static_cast<int>((oy[i] >> 22) & 0x1Fu);
          if (e0 + 4 * h + i < end && m < nvalid) {
            const int64_t slot = static_cast<int64_t>(ox[i]) * tr.Hkv + j;
            ws_logits[((slot * n_sel + (level - 1)) * G + g) * static_cast<int64_t>(CK) + r * kC + m] =
                c[i] * scale;
          }
        }
      }
    }
  }
}

static BucketArgs bucket_args(const recsa_tree& tr, void* ws, const WsLayout& w, int level) {
  char* b = static_cast<char*>(ws);
  BucketArgs ba;
  ba.tiles = reinterpret_cast<uint4*>(b + w.bk_tiles_off);
  ba.entries = reinterpret_cast<uint2*>(b + w.bk_entries_off);
  ba.n_tiles = reinterpret_cast<int32_t*>(b + w.bk_ntiles_off);
  ba.n_up = static_cast<int>(level_rows_host(tr.L_cap, level + 1) + 1);   // + the incomplete current node
  return ba;
}

// ------------------------------------------------------------- launchers
constexpr int64_t kTopkWideLists = 1024;   // below this many lists: 512-thread top-k

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
          bucket_clear_kernel<<<1, 64, 0, s>>>(ba);
          const unsigned nblk = static_cast<unsigned>(tr.B) *
                                static_cast<unsigned>((T + kFileQueries - 1) / kFileQueries);
          bucket_file_kernel<<<dim3(nblk, tr.Hkv), kBlock, 0, s>>>(tr, T, pos, sel, cnt, l,
                                                                  w.n_sel, ba);
          const int64_t wgs = (w.bk_max_tiles + kBlock / kWave - 1) / (kBlock / kWave);
          // a multiple of 8 workgroups (the tile walk splits them by XCD)
          const int64_t nwg = std::min<int64_t>((wgs + 7) / 8 * 8, 8192);
          bucket_score_kernel<D, G><<<static_cast<unsigned>(nwg), kBlock, 0, s>>>(
              tr, q, Hq, logits, l, w.n_sel, w.CK, ba);
          scored = true;
        }
      }
      if (!scored)
        score_kernel<DT, D, G><<<dim3(score_blocks * nq, tr.Hkv), kBlock, 0, s>>>(
            tr, q, Hq, T, pos, sel, cnt, logits, l, w.n_sel, w.CK);
    }
    // few lists (decode): 512 threads each, for the shortest latency; many
    // lists (prefill): 256, so more lists are resident per CU
    if (w.CK <= 4096 && static_cast<int64_t>(nq) * tr.Hkv < kTopkWideLists)
      topk_kernel<G, 2 * kBlock, 4096><<<dim3(nq, tr.Hkv), 2 * kBlock, 0, s>>>(
          tr, T, pos, sel, cnt, imp, logits, bitmap, l, w.n_sel, w.CK);
    else if (w.CK <= 4096)
      topk_kernel<G, kBlock, 4096><<<dim3(nq, tr.Hkv), kBlock, 0, s>>>(
          tr, T, pos, sel, cnt, imp, logits, bitmap, l, w.n_sel, w.CK);
    else
      topk_kernel<G, 2 * kBlock, kMaxCK><<<dim3(nq, tr.Hkv), 2 * kBlock, 0, s>>>(
          tr, T, pos, sel, cnt, imp, logits, bitmap, l, w.n_sel, w.CK);
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
  const dim3 grid(static_cast<unsigned>(n_split) * nq, tr.Hkv);
  const size_t sel_lds = static_cast<size_t>(w.n_sel) * (tr.k + 1) * sizeof(int32_t);
  if (decode)
    attn_kernel<DT, D, G, true><<<grid, kBlock, sel_lds, s>>>(
        tr, q, Hq, T, pos, const_cast<int32_t*>(sel), const_cast<int32_t*>(cnt), out, logits,
        bitmap, part, n_split, w.n_sel, w.CK);
  else
    attn_kernel<DT, D, G, false><<<grid, kBlock, sel_lds, s>>>(
        tr, q, Hq, T, pos, const_cast<int32_t*>(sel), const_cast<int32_t*>(cnt), out, logits,
        bitmap, part, n_split, w.n_sel, w.CK);
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
