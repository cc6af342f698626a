// Internal launcher declarations and workspace layout of librecsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "recsa.h"

namespace recsa {

__host__ __device__ __forceinline__ int64_t level_rows_dev(int64_t L_cap, int level) {
  return L_cap >> (4 * level);   // floor(L_cap / 16^level)
}
inline int64_t level_rows_host(int64_t L_cap, int level) { return L_cap >> (4 * level); }

// Workspace layout, per (query, KV head) "slot":
//   logits  [n_sel][G][C*k] float   (scored candidates' logits)
//   bitmap  [n_sel][C*k/32] uint32   (selected list positions)
// followed by the decode attention partials
//   part    [B][Hkv][n_split][G][d+2] float   (m, l, acc[d])
struct WsLayout {
  int n_sel, G, CK, d, n_split;
  int64_t slot_floats;        // logits floats per slot
  int64_t slot_words;         // bitmap words per slot
  int64_t n_slots;            // n_queries * Hkv
  int64_t logits_off, bitmap_off, part_off, total;   // bytes
};

inline WsLayout ws_layout(const recsa_tree& tr, int Hq, int64_t n_queries) {
  WsLayout w;
  w.n_sel = tr.n_levels > 1 ? tr.n_levels - 1 : 1;
  w.G = Hq / tr.Hkv;
  w.CK = tr.C * tr.k;
  w.d = tr.d;
  const int chunks_per_level = (w.CK + 255) / 256;
  w.n_split = w.n_sel * chunks_per_level;     // levels 0 .. n_levels-2
  w.slot_floats = static_cast<int64_t>(w.n_sel) * w.G * w.CK;
  w.slot_words = static_cast<int64_t>(w.n_sel) * ((w.CK + 31) / 32);
  w.n_slots = n_queries * tr.Hkv;
  w.logits_off = 0;
  w.bitmap_off = w.logits_off + w.n_slots * w.slot_floats * 4;
  w.part_off = w.bitmap_off + w.n_slots * w.slot_words * 4;
  w.part_off = (w.part_off + 255) & ~static_cast<int64_t>(255);
  const int64_t part = static_cast<int64_t>(tr.B) * tr.Hkv * w.n_split * w.G * (w.d + 2) * 4;
  w.total = w.part_off + part;
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
hipError_t launch_attn(const recsa_tree& tr, const void* q, int Hq, int T, const int64_t* pos,
                       const int32_t* sel, const int32_t* cnt, float* out, void* ws,
                       const WsLayout& w, bool decode, hipStream_t s);

}  // namespace recsa
