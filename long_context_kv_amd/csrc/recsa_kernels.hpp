// Internal launcher declarations and workspace layout of librecsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "recsa.h"
#include "recsa_common.hpp"

namespace recsa {

inline int64_t level_rows_host(int64_t L_cap, int level) { return L_cap >> (4 * level); }

// Workspace layout (bytes, 256-aligned regions):
//   logits  [n_queries*Hkv][n_sel][G][C*k] float   scored candidates' logits
//   bitmap  [n_queries*Hkv][n_sel][C*k/32] uint32  kept list positions
//   buckets (bf16, n_queries*Hkv >= kBucketMinSlots) multi-query scoring by
//           parent: tiles [max_tiles] uint4, entries [regions][kFileQueries*k]
//           uint2 (one region per filing workgroup), n_tiles int32
//   part    [B*Hkv][kPartSlots][G][4+d] float      decode attention partials
//           (max, sum, -, -, d values per query head)
//   ctl     [B*Hkv][kCtlWords] uint32              fused-decode control block:
//           word 1 = error word, words 16 + 16*w = arrival flag of workgroup w
// The ctl words must be zero before the first recsa_decode call; every call
// leaves them zero (except the error word, see recsa.h).
constexpr int kDecodeSplits = 64;    // attention workgroups per (query, KV head), decode
// most workgroups per query along the query launch dimension (scoring:
// C*k/64 <= 128 list blocks; decode attention: kDecodeSplits)
constexpr int kQueryLaunchX = 128;
constexpr int kPartSlots = kDecodeSplits > kFusedMaxW ? kDecodeSplits : kFusedMaxW;
constexpr int kCtlWords = 16 + 16 * kFusedMaxW;   // one 64-byte line per flag
constexpr int kBucketTile = 64;                   // bucket entries per scoring tile
constexpr int64_t kBucketMinSlots = 256;          // (query, KV head) slots from which
                                                  // bf16 scoring is bucketed by parent
constexpr int kFileQueries = 256;                 // queries per filing workgroup
constexpr int kFileMaxUp = 16384;                 // parents per (sequence, head) it bins in LDS

struct WsLayout {
  int n_sel, G, CK, d, n_split;
  int64_t n_slots;            // n_queries * Hkv
  int64_t logits_off, bitmap_off, part_off, ctl_off, total;   // bytes
  bool bucket;                // multi-query scoring by parent
  int64_t bk_regions, bk_max_tiles, bk_max_entries;
  int64_t bk_tiles_off, bk_entries_off, bk_ntiles_off;   // bytes
};

inline int64_t align256(int64_t x) { return (x + 255) & ~static_cast<int64_t>(255); }

inline WsLayout ws_layout(const recsa_tree& tr, int Hq, int64_t n_queries) {
  WsLayout w;
  w.n_sel = tr.n_levels > 1 ? tr.n_levels - 1 : 1;
  w.G = Hq / tr.Hkv;
  w.CK = tr.C * tr.k;
  w.d = tr.d;
  w.n_split = kDecodeSplits;
  w.n_slots = n_queries * tr.Hkv;
  const int64_t slot_floats = static_cast<int64_t>(w.n_sel) * w.G * w.CK;
  const int64_t slot_words = static_cast<int64_t>(w.n_sel) * ((w.CK + 31) / 32);
  const int64_t heads = static_cast<int64_t>(tr.B) * tr.Hkv;
  w.logits_off = 0;
  w.bitmap_off = align256(w.logits_off + w.n_slots * slot_floats * 4);
  int64_t end = w.bitmap_off + w.n_slots * slot_words * 4;
  // parents of level-1 lists (the longest): nodes 0 .. N_2 of level 2 (node
  // N_2 may be the incomplete current node, whose complete children are
  // still scored).  Filing workgroups: at most n_queries/kFileQueries + B per
  // KV head (blocks of one sequence), each with a region of kFileQueries*k
  // entries (<= k parents per query) and at most one partial tile per parent.
  const int64_t n_up = level_rows_host(tr.L_cap, 2) + 1;
  w.bk_regions = (n_queries / kFileQueries + tr.B) * tr.Hkv;
  w.bk_max_entries = w.bk_regions * kFileQueries * tr.k;
  w.bk_max_tiles =
      w.bk_regions * (std::min<int64_t>(n_up, int64_t{kFileQueries} * tr.k) +
                      int64_t{kFileQueries} * tr.k / kBucketTile);
  w.bucket = tr.dtype == RECSA_BF16 && tr.n_levels >= 3 && w.n_slots >= kBucketMinSlots &&
             n_up <= kFileMaxUp && w.bk_max_entries < (int64_t{1} << 32) &&
             w.bk_max_tiles < (int64_t{1} << 31) && n_queries < (int64_t{1} << 31);
  w.bk_tiles_off = w.bk_entries_off = w.bk_ntiles_off = 0;
  if (w.bucket) {
    w.bk_tiles_off = align256(end);
    w.bk_entries_off = align256(w.bk_tiles_off + w.bk_max_tiles * 16);
    w.bk_ntiles_off = align256(w.bk_entries_off + w.bk_max_entries * 8);
    end = w.bk_ntiles_off + 4;
  }
  w.part_off = align256(end);
  w.ctl_off = align256(w.part_off + heads * kPartSlots * w.G * (w.d + kPartHead) * 4);
  w.total = w.ctl_off + heads * kCtlWords * 4;   // the control words end the workspace
  return w;
}

hipError_t launch_rope_table(float* table, int d, int n_pos, double theta, hipStream_t s);
hipError_t launch_build(const recsa_tree& tr, const recsa_pooler& P, int64_t tb, int64_t te,
                        hipStream_t s);
hipError_t launch_append(const recsa_tree& tr, const recsa_pooler& P, const void* k_new,
                         const void* v_new, const int64_t* pos, hipStream_t s);
hipError_t launch_select(const recsa_tree& tr, const void* q, int Hq, int T, const int64_t* pos,
                         int32_t* sel, int32_t* cnt, float* imp, void* ws, const WsLayout& w,
                         hipStream_t s);
hipError_t launch_decode_fused(const recsa_tree& tr, const recsa_pooler& P, const void* k_new,
                               const void* v_new, const void* q, int Hq, const int64_t* pos,
                               int32_t* sel, int32_t* cnt, float* out, void* ws, const WsLayout& w,
                               hipStream_t s);
hipError_t launch_attn(const recsa_tree& tr, const void* q, int Hq, int T, const int64_t* pos,
                       const int32_t* sel, const int32_t* cnt, float* out, void* ws,
                       const WsLayout& w, bool decode, hipStream_t s);

// Pooler distillation losses (Eq. 6, Eq. 7)
int64_t distill_groups(int64_t L_cap);
int64_t distill_ws_bytes(const recsa_tree& tr, int Hq, int64_t n_queries);
hipError_t launch_distill_kl(const recsa_tree& tr, const void* q, int Hq, int T,
                             const int64_t* pos, const int32_t* sel, const int32_t* cnt,
                             const float* imp, double theta, float* kl, float* y, void* ws,
                             hipStream_t s);
int64_t shift_ws_bytes(const recsa_tree& tr);
hipError_t launch_shift_penalty(const recsa_tree& tr, const recsa_pooler& P, int64_t tok_end,
                                float* out, void* ws, hipStream_t s);

// Gradient of the Eq. 6 terms with respect to the node keys
int64_t kgrad_ws_bytes(const recsa_tree& tr, int Hq, int64_t n_queries);
int64_t kgrad_out_floats(const recsa_tree& tr);
hipError_t launch_kgrad(const recsa_tree& tr, const void* q, int Hq, int T, const int64_t* pos,
                        const int32_t* sel, const int32_t* cnt, const float* imp,
                        const float* teacher, const float* logits, float* dK, void* ws,
                        hipStream_t s);

// Pooler backward (Eq. 5 VJP)
int64_t pool_bwd_ws_bytes(const recsa_tree& tr, const recsa_pooler& P, int level);
hipError_t launch_pool_backward(const recsa_tree& tr, const recsa_pooler& P, int level,
                                int64_t tok_end, const float* dK, const float* shift_sums,
                                float shift_weight, const recsa_pooler_grad& G, void* ws,
                                hipStream_t s);

#define RECSA_DISPATCH(FN, ...)                                                     \
  do {                                                                              \
    const int G = Hq / tr.Hkv;                                                      \
    if (tr.dtype == RECSA_BF16 && tr.d == 128) {                                    \
      if (G == 4) return FN<RECSA_BF16, 128, 4>(__VA_ARGS__);                       \
      if (G == 1) return FN<RECSA_BF16, 128, 1>(__VA_ARGS__);                       \
      if (G == 2) return FN<RECSA_BF16, 128, 2>(__VA_ARGS__);                       \
    } else if (tr.dtype == RECSA_BF16 && tr.d == 64) {                              \
      if (G == 4) return FN<RECSA_BF16, 64, 4>(__VA_ARGS__);                        \
      if (G == 1) return FN<RECSA_BF16, 64, 1>(__VA_ARGS__);                        \
      if (G == 2) return FN<RECSA_BF16, 64, 2>(__VA_ARGS__);                        \
    } else if (tr.dtype == RECSA_F32 && tr.d == 128) {                              \
      if (G == 4) return FN<RECSA_F32, 128, 4>(__VA_ARGS__);                        \
      if (G == 1) return FN<RECSA_F32, 128, 1>(__VA_ARGS__);                        \
      if (G == 2) return FN<RECSA_F32, 128, 2>(__VA_ARGS__);                        \
    } else if (tr.dtype == RECSA_F32 && tr.d == 64) {                               \
      if (G == 4) return FN<RECSA_F32, 64, 4>(__VA_ARGS__);                         \
      if (G == 1) return FN<RECSA_F32, 64, 1>(__VA_ARGS__);                         \
      if (G == 2) return FN<RECSA_F32, 64, 2>(__VA_ARGS__);                         \
    }                                                                               \
    return hipErrorInvalidValue;                                                    \
  } while (0)

}  // namespace recsa
