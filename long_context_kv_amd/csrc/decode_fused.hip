// One decode step -- append, hierarchical selection (picx.dev Hierarchical
// Selection, Eq. 3) and the unified softmax (Unified Softmax, Eq. 4) -- in
// one persistent launch.
//
// 1-D grid of W * S workgroups of 512 threads; workgroup id = w * S + g
// serves (sequence, KV head) group g < B * Hkv as its member w (ids with
// g >= B * Hkv exit at once).  The W workgroups of a group cooperate:
//   WG 0 appends token t (row t, and every node whose last token is t: those
//   are current nodes of this query, never read by it);
//   for each level from the top down that must be scored: the W workgroups
//   score interleaved groups of the candidate list into the workspace, meet
//   at a barrier, and then every workgroup runs the same exact top-(k-1) on
//   all the logits, keeping S and the kept-position bitmap in its own LDS
//   (WG 0 also writes them out), so no second barrier is needed;
//   all W then accumulate interleaved entry chunks (token t's row comes from
//   k_new/v_new), publish a partial softmax state, and WG 0 waits for them
//   and merges them into the output.
// Barriers come in two forms.  XCD-local: the device hands the workgroups of
// a dispatch to its XCDs round-robin, workgroup i to XCD (i + s) mod n_xcd
// for an offset s that varies between dispatches (graph replays start at
// other XCDs than direct launches), so with S a multiple of n_xcd all
// workgroups of a group share one XCD and its L2; arrivals are atomic adds on
// one counter in that L2 and waits read it with an L2 atomic, with no L2
// write-back or invalidation.  Each workgroup also ORs its XCD id into a
// placement mask with a device-scope atomic; the merging workgroup checks
// that the group's mask names a single XCD.  Device-wide:
// per-workgroup flags raised and polled with device-scope atomics around
// release/acquire fences.  Either way every wait is a bounded spin; if the
// bound is hit the error word is set and the output is poisoned with NaN.
// The host launches this kernel only when the grid fits on the device (on
// each XCD, for the local form) with room to spare.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "recsa_common.hpp"
#include "recsa_device.hpp"
#include "recsa_fused_ctl.hpp"
#include "recsa_mfma.hpp"
#include "recsa_kernels.hpp"
#include "recsa_pool.hpp"

namespace recsa {

constexpr int kFusedThreads = 512;
// Merge the W partial softmax states [W][G][kPartHead + D] (max, sum, -,
// -, weighted values) of one group into the output [G][D].  Thread (column
// c, subset q) owns the 4 output values 4c..4c+3 over the partials w = q,
// q + NQ, ...: it issues those loads (values and normaliser) first, while
// the first W*G threads bring every partial's maximum into LDS; after one
// barrier each thread forms its head's maximum, its partials' weights and
// their share of the normaliser, and after a second the threads of subset
// 0 add the NQ shares and write the output.
template <int D, int G, int NT>
__device__ void merge_partials_fused(const float* __restrict__ pp, int W, float* __restrict__ o) {
  constexpr int PS = D + kPartHead;                  // floats per query head of a partial
  constexpr int stride = G * PS;
  constexpr int NC = G * D / 4;                      // float4 columns of the output
  static_assert(NT % NC == 0 && NT >= kFusedMaxW * kMaxG, "thread count");
  constexpr int NQ = NT / NC;                        // partial subsets
  constexpr int WQ = (kFusedMaxW + NQ - 1) / NQ;     // partials per thread
  __shared__ float s_m[kMaxG][kFusedMaxW];
  __shared__ float4 s_acc[NQ][NC];
  __shared__ float s_l[NQ][NC];
  const int tid = threadIdx.x;
  const int c = tid % NC, qs = tid / NC;
  const int ge = (4 * c) / D, dd = (4 * c) % D;
  const float* ph = pp + ge * PS;                    // this head's state in partial 0
  float4 av[WQ];
  float lw[WQ];
#pragma unroll
  for (int i = 0; i < WQ; ++i) {
    const int w = qs + NQ * i;
    av[i] = w < W ? *reinterpret_cast<const float4*>(ph + w * stride + kPartHead + dd)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    lw[i] = w < W ? ph[w * stride + 1] : 0.f;
  }
  if (tid < W * G) {
    const int w = tid / G, g = tid % G;
    s_m[g][w] = pp[w * stride + g * PS];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int v = 0; v < W; ++v) M = fmaxf(M, s_m[ge][v]);
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
#pragma unroll
  for (int i = 0; i < WQ; ++i) {
    const int w = qs + NQ * i;
    if (w < W) {
      const float mv = s_m[ge][w];
      const float f = (mv == -INFINITY) ? 0.f : __expf(mv - M);
      a.x += f * av[i].x;
      a.y += f * av[i].y;
      a.z += f * av[i].z;
      a.w += f * av[i].w;
      L += f * lw[i];
    }
  }
  s_acc[qs][c] = a;
  s_l[qs][c] = L;
  __syncthreads();
  if (qs == 0) {
    float4 r = s_acc[0][c];
    float l = s_l[0][c];
#pragma unroll
    for (int q2 = 1; q2 < NQ; ++q2) {
      const float4 x = s_acc[q2][c];
      r.x += x.x; r.y += x.y; r.z += x.z; r.w += x.w;
      l += s_l[q2][c];
    }
    const float inv = 1.0f / l;
    *reinterpret_cast<float4*>(o + 4 * c) = make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
  }
}

// CKM: the top-k's list-size class (C*k <= CKM); each class is its own
// kernel, so the one top-k it holds is inlined and the kernel makes no calls
// (no private stack for the dispatch to set up).
template <int DT, int D, int G, bool XL, int CKM>
__global__ void __launch_bounds__(kFusedThreads)
    decode_fused_kernel(recsa_tree tr, recsa_pooler P, const void* k_new, const void* v_new,
                        const void* q, int Hq, const int64_t* pos, int32_t* sel, int32_t* cnt,
                        float* out, float* ws_logits, float* part, uint32_t* ctl_words, int W,
                        int S, int n_xcd, int n_sel, int CK) {
  using T = typename Stor<DT>::T;
  constexpr int NT = kFusedThreads;
  constexpr int NW = NT / kWave;
  constexpr int kMaxSel = RECSA_MAX_LEVELS - 1;
  // S^(l) of every level for this group, level l at [(l-1)*k, l*k) -- the
  // stride list_view reads the parent selection with (k <= kMaxK)
  __shared__ int32_t s_sel[kMaxSel * kMaxK];
  __shared__ int32_t s_cnt[kMaxSel + 1];
  __shared__ uint32_t s_bm[kMaxSel * (CKM / 32)];
  __shared__ uint32_t s_fail;
  __shared__ float qs[G * D];
  __shared__ union Smem {
    TopkSmem tk;
    AttnSmem<D, G, NT> at;
    PoolSmem<DT, D, 1> pl;
  } sm;
  const int grp = static_cast<int>(blockIdx.x) % S, w = static_cast<int>(blockIdx.x) / S;
  if (grp >= tr.B * tr.Hkv) return;                  // padding of the group stride
  const int j = grp % tr.Hkv, b = grp / tr.Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid >> 6;
  const int k = tr.k;
  const int top = tr.n_levels - 1;
  const int bm_words = (CK + 31) / 32;
  const int64_t slot = static_cast<int64_t>(b) * tr.Hkv + j;    // one query per sequence
  const int64_t t = pos[b];
  int32_t* sel_q = sel + slot * n_sel * k;
  int32_t* cnt_q = cnt + slot * n_sel;
  float* lg_slot = ws_logits + slot * n_sel * static_cast<int64_t>(G) * CK;
  const FusedCtl ctl = fused_ctl(ctl_words + slot * kCtlWords);
  const T* k_t = static_cast<const T*>(k_new) + slot * D;
  const T* v_t = static_cast<const T*>(v_new) + slot * D;
  if (tid == 0) {
    s_fail = 0u;
    // the local barrier needs every workgroup of the group on one XCD:
    // record this one's XCD in the group's placement mask (no wait for the
    // atomic: its round trip overlaps the query loads)
    if constexpr (XL) ctl_mark_xcd_post(ctl);
  }
  load_query_rows<DT, D, G, NT>(q, static_cast<int64_t>(b) * Hq + static_cast<int64_t>(j) * G, qs);

  // ---- append (WG 0)
  if (w == 0) {
    T* kd = static_cast<T*>(tr.K[0]) + (slot * tr.L_cap + t) * D;
    T* vd = static_cast<T*>(tr.V[0]) + (slot * tr.L_cap + t) * D;
    for (int i = tid; i < D; i += NT) {
      kd[i] = k_t[i];
      vd[i] = v_t[i];
    }
    if (tr.Kr[0])
      rotate_key_row<DT, D>(k_t, static_cast<T*>(tr.Kr[0]) + (slot * tr.L_cap + t) * D,
                            static_cast<int>(t % kC), tr.rope, tid, NT);
    int64_t span = 1;
    for (int l = 1; l < tr.n_levels; ++l) {
      span *= kC;
      if ((t + 1) % span != 0) break;
      __threadfence();
      __syncthreads();
      const int64_t node = (t + 1) / span - 1;
      const int64_t rows_up = level_rows_dev(tr.L_cap, l - 1);
      const int64_t rows = level_rows_dev(tr.L_cap, l);
      pool_tile<DT, D, 1, NT>(static_cast<const T*>(tr.K[l - 1]) + (slot * rows_up + node * kC) * D,
                              static_cast<const T*>(tr.V[l - 1]) + (slot * rows_up + node * kC) * D,
                              static_cast<T*>(tr.K[l]) + (slot * rows + node) * D,
                              static_cast<T*>(tr.V[l]) + (slot * rows + node) * D,
                              tr.Kr[l] ? static_cast<T*>(tr.Kr[l]) + (slot * rows + node) * D
                                       : nullptr,
                              static_cast<int>(node % kC), tr.rope, 1, P, sm.pl);
      __syncthreads();
    }
    if (top >= 1) {                    // the top list [0 .. a_top] is fully selected
      const ListView lt = list_view(t, top, top, k, sel_q, cnt_q);
      wg_take_all<NT>(lt, k, sel_q + static_cast<int64_t>(top - 1) * k, cnt_q + (top - 1), nullptr, CK);
    }
  }
  __syncthreads();

  // ---- selection, top level down (S^(l) kept in LDS by every workgroup)
  uint32_t gen = 0;
  for (int l = top - 1; l >= 1; --l) {
    const ListView lv = list_view(t, l, top, k, s_sel, s_cnt);
    int32_t* ls = s_sel + (l - 1) * k;
    if (lv.len <= k) {
      wg_take_all<NT>(lv, k, ls, s_cnt + (l - 1), nullptr, CK);
    } else {
      const int n = lv.len - 1;
      const int ng = (n + kC - 1) / kC;
      const int64_t rows_l = level_rows_dev(tr.L_cap, l);
      const int p_q = lv.len - 1;
      float* out_l = lg_slot + static_cast<int64_t>(l - 1) * G * CK;
      // at the first scored level workgroup 0 has spent the start appending,
      // so the other W - 1 take its share of the groups
      const bool skip0 = gen == 0 && W > 1;
      const int wl = skip0 ? w - 1 : w, Wl = skip0 ? W - 1 : W;
      for (int gi = wl + Wl * wid; wl >= 0 && gi < ng; gi += Wl * NW) {
        const int p0 = gi * kC;
        const int nvalid = min(kC, n - p0);
        const bool raw = tr.Kr[l] == nullptr;     // no rotated copy: rotate the rows here
        const T* rows = static_cast<const T*>(raw ? tr.K[l] : tr.Kr[l]) +
                        (slot * rows_l + lv.node(p0)) * D;
        const int phi = p_q - p0;        // = C (r_q - r) + c_q, r = p0 / C
        if constexpr (DT == RECSA_BF16) {
          // the table row first (the rotation waits only for it), then the
          // key rows, in flight during the rotation
          MFrag<D> kf, qf;
          QRope<DT, D, G> rq;
          load_query_rope<DT, D, G>(phi, tr.rope, rq);
          load_key_frag<D>(rows, nvalid, kf);
          rotate_query_from<DT, D, G>(qs, sm.at.qt[wid], rq);
          if (raw) rotate_key_frag<D>(kf, tr.rope);
          wave_sync();
          query_frag_lds<D, G>(reinterpret_cast<const uint16_t*>(sm.at.qt[wid]), qf);
          const f32x4_t c = mfma_logits<D>(qf, kf);
          store_logit_tile<D, G>(c, out_l, CK, p0, nvalid);
        } else {
          KRows<DT, D> kr;               // key rows in flight during the rotation
          QRope<DT, D, G> rq;
          load_query_rope<DT, D, G>(phi, tr.rope, rq);
          group_load_k<DT, D>(rows, 0, nvalid, kr);
          rotate_query_from<DT, D, G>(qs, sm.at.qt[wid], rq);
          wave_sync();
          float lg[G];
          group_logits_any<DT, D, G>(raw, kr, 0, nvalid, sm.at.qt[wid], tr.rope, lg);
          const int c = lane >> 2, s = lane & 3;
          if (c < nvalid) {
#pragma unroll
            for (int g = 0; g < G; ++g)
              if ((g & 3) == s) out_l[static_cast<int64_t>(g) * CK + p0 + c] = lg[g];
          }
        }
        wave_sync();
      }
      ++gen;
      if constexpr (XL)
        group_barrier_xcd(ctl.counter, gen * static_cast<uint32_t>(W), ctl.err, &s_fail);
      else
        group_barrier(ctl.flags, w, W, gen, ctl.err, &s_fail);
      wg_topk<G, NT, CKM>(out_l, n, k, CK, lv, ls, s_cnt + (l - 1), s_bm + (l - 1) * bm_words,
                          nullptr, sm.tk);
    }
    __syncthreads();
    if (w == 0) {                      // API outputs
      for (int i = tid; i < k; i += NT) sel_q[static_cast<int64_t>(l - 1) * k + i] = ls[i];
      if (tid == 0) cnt_q[l - 1] = s_cnt[l - 1];
    }
  }

  // ---- unified softmax over this workgroup's interleaved entry groups
  const EntryGroups eg = entry_groups(t, tr, n_sel, s_sel, s_cnt);
  // two-group level-0 chunks and four-group summary chunks (as many
  // registers per wave, no spills): at the longest lists about one chunk
  // per wave, so the group's loads go out in one round
  // (the waves' merge writes this workgroup's partial state straight out)
  float* pp = part + (slot * kPartSlots + w) * static_cast<int64_t>(G) * (D + kPartHead);
  attn_groups<DT, D, G, NT, 2, true>(tr, t, slot, s_sel, s_cnt, eg, w, W, qs, lg_slot, s_bm, CK,
                                     k_t, v_t, sm.at, pp);
  float* o = out + (static_cast<int64_t>(b) * Hq + static_cast<int64_t>(j) * G) * D;
  const float* pp_group = part + slot * kPartSlots * static_cast<int64_t>(G) * (D + kPartHead);
  // s_fail is only written inside the waits, each of which ends with a
  // workgroup barrier, so every thread reads its final value here
  if (s_fail) {
    // one of this workgroup's waits timed out: its selection and partial may
    // be built on incomplete data, and the merge may never run (members on
    // two XCDs count in two L2s), so it poisons the output itself; the error
    // word is already set
    for (int e = tid; e < G * D; e += NT) o[e] = __builtin_nanf("");
  }
  if constexpr (XL) {
    // ---- the last workgroup to arrive merges (its arrival completes the
    // count, so every partial is in the L2); the others are done
    __shared__ uint32_t s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the group's status words are read by the merging thread as soon as
    // it knows every member has arrived and first used after the merge, so
    // their latency overlaps it
    FusedStatus st;
    if (tid == 0) s_last = xl_final_arrival(ctl, gen, W, st) ? 1u : 0u;
    __syncthreads();
    if (!s_last) return;
    merge_partials_fused<D, G, NT>(pp_group, W, o);
    __shared__ uint32_t s_bad;
    if (tid == 0) s_bad = xl_result_bad(ctl, st, s_fail) ? 1u : 0u;
    __syncthreads();
    if (s_bad) {
      for (int e = tid; e < G * D; e += NT) o[e] = __builtin_nanf("");
    }
    if (tid == 0) xl_reset(ctl);
  } else {
    // ---- WG 0 waits for every partial and merges them
    if (w != 0) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) dw_final_flag(ctl, w, gen);
      return;
    }
    group_barrier(ctl.flags, w, W, gen + 1, ctl.err, &s_fail);
    merge_partials_fused<D, G, NT>(pp_group, W, o);
    __syncthreads();
    if (dw_result_bad(ctl, s_fail)) {
      for (int e = tid; e < G * D; e += NT) o[e] = __builtin_nanf("");
    }
    // every other workgroup has raised its final flag, so none reads them again
    dw_reset(ctl, tid, W);
  }
}


// Largest W such that B*Hkv*W workgroups are resident at once (0: none fit).
// Launch geometry of one decode step.
struct FusedGeom {
  int W = 0;          // workgroups per (sequence, KV head)
  int S = 0;          // group stride of the workgroup id
  int n_xcd = 1;
  bool xl = false;    // XCD-local barrier
};

// Device facts, cached per device: CUs, co-resident workgroups per CU for
// both forms of the kernel, and the XCD count when the device is known to
// hand out workgroups to its XCDs round-robin (gfx950: 32 CUs per XCD).
template <int DT, int D, int G, int CKM>
static FusedGeom fused_geom(const recsa_tree& tr) {
  static int cached_dev = -1, cus = 0, per_cu_xl = 0, per_cu = 0, n_xcd = 0;
  int dev = 0;
  FusedGeom g;
  if (hipGetDevice(&dev) != hipSuccess) return g;
  if (dev != cached_dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return g;
    cus = prop.multiProcessorCount;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, decode_fused_kernel<DT, D, G, false, CKM>, kFusedThreads, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu_xl, decode_fused_kernel<DT, D, G, true, CKM>, kFusedThreads, 0) != hipSuccess)
      return g;
    n_xcd = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 && cus % 32 == 0) ? cus / 32 : 0;
    const char* env = std::getenv("RECSA_FUSED_XCD_LOCAL");
    if (env && env[0] == '0') n_xcd = 0;
    cached_dev = dev;
  }
  const int64_t groups = static_cast<int64_t>(tr.B) * tr.Hkv;
  // keep part of the capacity spare so a group never waits on a workgroup
  // that cannot be placed (an eighth of each XCD; a quarter of the device)
  if (n_xcd > 0) {
    const int64_t S = (groups + n_xcd - 1) / n_xcd * n_xcd;
    const int64_t cap = static_cast<int64_t>(cus / n_xcd) * per_cu_xl * 7 / 8;
    g.W = static_cast<int>(std::min<int64_t>(kFusedMaxW, cap / (S / n_xcd)));
    g.S = static_cast<int>(S);
    g.n_xcd = n_xcd;
    g.xl = true;
  } else {
    const int64_t cap = static_cast<int64_t>(cus) * per_cu * 3 / 4;
    g.W = static_cast<int>(std::min<int64_t>(kFusedMaxW, cap / groups));
    g.S = static_cast<int>(groups);
  }
  return g;
}

template <int DT, int D, int G, int CKM>
static hipError_t fused_launch(const recsa_tree& tr, const recsa_pooler& P, const void* k_new,
                               const void* v_new, const void* q, int Hq, const int64_t* pos,
                               int32_t* sel, int32_t* cnt, float* out, void* ws,
                               const WsLayout& w, hipStream_t s) {
  const FusedGeom g = fused_geom<DT, D, G, CKM>(tr);
  if (g.W < 1) return hipErrorLaunchOutOfResources;
  char* base = static_cast<char*>(ws);
  const dim3 grid(static_cast<unsigned>(g.W) * static_cast<unsigned>(g.S));
  float* lg = reinterpret_cast<float*>(base + w.logits_off);
  float* part = reinterpret_cast<float*>(base + w.part_off);
  uint32_t* ctl = reinterpret_cast<uint32_t*>(base + w.ctl_off);
  if (g.xl)
    decode_fused_kernel<DT, D, G, true, CKM><<<grid, kFusedThreads, 0, s>>>(
        tr, P, k_new, v_new, q, Hq, pos, sel, cnt, out, lg, part, ctl, g.W, g.S, g.n_xcd, w.n_sel,
        w.CK);
  else
    decode_fused_kernel<DT, D, G, false, CKM><<<grid, kFusedThreads, 0, s>>>(
        tr, P, k_new, v_new, q, Hq, pos, sel, cnt, out, lg, part, ctl, g.W, g.S, g.n_xcd, w.n_sel,
        w.CK);
  return hipGetLastError();
}

template <int DT, int D, int G>
static hipError_t fused_impl(const recsa_tree& tr, const recsa_pooler& P, const void* k_new,
                             const void* v_new, const void* q, int Hq, const int64_t* pos,
                             int32_t* sel, int32_t* cnt, float* out, void* ws, const WsLayout& w,
                             hipStream_t s) {
  if (w.CK <= 4096)
    return fused_launch<DT, D, G, 4096>(tr, P, k_new, v_new, q, Hq, pos, sel, cnt, out, ws, w, s);
  return fused_launch<DT, D, G, kMaxCK>(tr, P, k_new, v_new, q, Hq, pos, sel, cnt, out, ws, w, s);
}

hipError_t launch_decode_fused(const recsa_tree& tr, const recsa_pooler& P, const void* k_new,
                               const void* v_new, const void* q, int Hq, const int64_t* pos,
                               int32_t* sel, int32_t* cnt, float* out, void* ws, const WsLayout& w,
                               hipStream_t s) {
  RECSA_DISPATCH(fused_impl, tr, P, k_new, v_new, q, Hq, pos, sel, cnt, out, ws, w, s);
}

}  // namespace recsa
