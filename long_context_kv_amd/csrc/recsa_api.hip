// C ABI of librecsa: argument validation, then stream-ordered launches.
// Nothing is launched when validation fails; no call allocates, frees or
// synchronises, so every call can be captured into a HIP graph.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "recsa_common.hpp"
#include "recsa_kernels.hpp"

using namespace recsa;

// Workspace of recsa_decode_static: one array per device, held until the
// process ends.  Host code never uses this name as an address; it takes the
// device address from hipGetSymbolAddress once per device.
constexpr size_t kStaticScratchBytes = size_t{32} << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

// Arrays of float32 or bf16 values are read and written with 16-byte vector
// accesses, so they must be 16-byte aligned (HIP and torch allocations are
// 256-byte aligned, and so is every whole-row slice of them); index arrays
// need their element's alignment.  NULL passes: presence is checked apart.
bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool a8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool a4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool tree_ok(const recsa_tree* t, int* why) {
  *why = RECSA_E_INVALID;
  if (!t) return false;
  if (t->B < 1 || t->Hkv < 1 || t->L_cap < 1 || t->k < 1 || t->n_levels < 1 ||
      t->n_levels > RECSA_MAX_LEVELS)
    return false;
  if (t->dtype != RECSA_F32 && t->dtype != RECSA_BF16) { *why = RECSA_E_UNSUPPORTED; return false; }
  if (t->C != kC || (t->d != 64 && t->d != 128) || t->k > kMaxK ||
      static_cast<int64_t>(t->C) * t->k > kMaxCK) {
    *why = RECSA_E_UNSUPPORTED;
    return false;
  }
  if (t->L_cap > (int64_t{1} << 40)) return false;
  if (t->n_levels < recsa_levels_needed(t->L_cap, t->C, t->k)) return false;
  if (!t->rope || !a16(t->rope)) return false;
  // the rotated-key copy Kr is optional, but all or nothing
  const bool has_kr = t->Kr[0] != nullptr;
  for (int l = 0; l < t->n_levels; ++l) {
    if (level_rows_host(t->L_cap, l) > 0 &&
        (!t->K[l] || !t->V[l] || (has_kr != (t->Kr[l] != nullptr))))
      return false;
    if (!a16(t->K[l]) || !a16(t->V[l]) || !a16(t->Kr[l])) return false;
  }
  return true;
}

bool pooler_ok(const recsa_pooler* p, const recsa_tree* t) {
  if (!p) return false;
  if (p->d != t->d || p->hidden < 16 || p->hidden > 256 || p->hidden % 16 != 0) return false;
  if (!p->w || !p->W1 || !p->b1 || !p->W2) return false;
  if (!a16(p->w) || !a16(p->W1) || !a16(p->b1) || !a16(p->W2)) return false;
  if (!isfinite(p->tau) || !isfinite(p->g) || !isfinite(p->eps) || p->eps < 0.f) return false;
  return true;
}

// Query heads per KV head: 1, 2 or 4.  (8 is switched off: the one GPU run
// of its fused decode failed, and no cause has been shown; its build needs
// 256 VGPRs with a 76-byte spill and 119 KB of LDS per workgroup.)
bool heads_ok(const recsa_tree* t, int32_t Hq) {
  if (Hq < 1 || Hq % t->Hkv != 0) return false;
  const int G = Hq / t->Hkv;
  return G == 1 || G == 2 || G == 4;
}

// B*T queries, each launched as up to kQueryLaunchX workgroups along one grid
// dimension, and B*T*Hkv selection slots, all within 31 bits.
bool queries_fit(const recsa_tree* t, int32_t T) {
  const int64_t nq = static_cast<int64_t>(t->B) * T;
  return nq * kQueryLaunchX <= 0x7FFFFFFF && nq * t->Hkv <= 0x7FFFFFFF;
}

int hip_status(hipError_t e) { return e == hipSuccess ? RECSA_OK : RECSA_E_HIP; }

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Zero n 32-bit words (a kernel, not a memset node, so the call stays safe to
// capture into a graph).
__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

}  // namespace

extern "C" {

const char* recsa_status_string(int status) {
  switch (status) {
    case RECSA_OK: return "ok";
    case RECSA_E_INVALID: return "invalid argument";
    case RECSA_E_UNSUPPORTED: return "unsupported configuration";
    case RECSA_E_WORKSPACE: return "workspace too small";
    case RECSA_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int64_t recsa_level_rows(int64_t L_cap, int32_t C, int32_t level) {
  if (L_cap < 0 || C < 2 || level < 0) return 0;
  int64_t r = L_cap;
  for (int l = 0; l < level && r > 0; ++l) r /= C;
  return r;
}

int32_t recsa_levels_needed(int64_t L_cap, int32_t C, int32_t k) {
  if (L_cap < 1 || C < 2 || k < 1) return 0;
  const int64_t t_max = L_cap - 1;
  int32_t D = 1;
  int64_t span = 1;
  while (t_max / span + 1 > k) {
    span *= C;
    ++D;
  }
  return D;
}

int recsa_init_rope(float* table, int32_t d, int32_t n_pos, double theta, void* stream) {
  if (!table || !a16(table) || d < 2 || d % 2 != 0 || n_pos < 1 || !(theta > 1.0))
    return RECSA_E_INVALID;
  return hip_status(launch_rope_table(table, d, n_pos, theta, static_cast<hipStream_t>(stream)));
}

size_t recsa_workspace_bytes(const recsa_tree* tree, int32_t Hq, int64_t n_queries) {
  int why;
  if (!tree_ok(tree, &why) || !heads_ok(tree, Hq) || n_queries < 1) return 0;
  return static_cast<size_t>(ws_layout(*tree, Hq, n_queries).total);
}

int recsa_build_tree(const recsa_tree* tree, const recsa_pooler* pooler, int64_t tok_begin,
                     int64_t tok_end, void* stream) {
  int why;
  if (!tree_ok(tree, &why)) return why;
  if (!pooler_ok(pooler, tree)) return RECSA_E_INVALID;
  if (tok_begin < 0 || tok_end < tok_begin || tok_end > tree->L_cap) return RECSA_E_INVALID;
  if (tok_end == tok_begin) return RECSA_OK;
  return hip_status(launch_build(*tree, *pooler, tok_begin, tok_end, static_cast<hipStream_t>(stream)));
}

int recsa_append_decode(const recsa_tree* tree, const recsa_pooler* pooler, const void* k_new,
                        const void* v_new, const int64_t* pos_dev, void* stream) {
  int why;
  if (!tree_ok(tree, &why)) return why;
  if (!pooler_ok(pooler, tree) || !k_new || !v_new || !pos_dev) return RECSA_E_INVALID;
  if (!a16(k_new) || !a16(v_new) || !a8(pos_dev)) return RECSA_E_INVALID;
  return hip_status(launch_append(*tree, *pooler, k_new, v_new, pos_dev, static_cast<hipStream_t>(stream)));
}

int recsa_select(const recsa_tree* tree, const void* q, int32_t Hq, int32_t T, const int64_t* pos_dev,
                 int32_t* sel_idx, int32_t* sel_cnt, float* importance_or_null, void* ws,
                 size_t ws_bytes, void* stream) {
  int why;
  if (!tree_ok(tree, &why)) return why;
  if (!heads_ok(tree, Hq)) return RECSA_E_UNSUPPORTED;
  if (!q || T < 1 || !pos_dev || !sel_idx || !sel_cnt || !ws) return RECSA_E_INVALID;
  if (!a16(q) || !a8(pos_dev) || !a4(sel_idx) || !a4(sel_cnt) || !a16(importance_or_null) ||
      !a16(ws))
    return RECSA_E_INVALID;
  if (!queries_fit(tree, T)) return RECSA_E_INVALID;
  const WsLayout w = ws_layout(*tree, Hq, static_cast<int64_t>(tree->B) * T);
  if (ws_bytes < static_cast<size_t>(w.total)) return RECSA_E_WORKSPACE;
  if (tree->n_levels < 2) return RECSA_OK;      // a single level: nothing to select
  return hip_status(launch_select(*tree, q, Hq, T, pos_dev, sel_idx, sel_cnt, importance_or_null,
                                  ws, w, static_cast<hipStream_t>(stream)));
}

static int attn_common(const recsa_tree* tree, const void* q, int32_t Hq, int32_t T,
                       const int64_t* pos_dev, const int32_t* sel_idx, const int32_t* sel_cnt,
                       float* out, void* ws, size_t ws_bytes, bool decode, void* stream) {
  int why;
  if (!tree_ok(tree, &why)) return why;
  if (!heads_ok(tree, Hq)) return RECSA_E_UNSUPPORTED;
  if (!q || T < 1 || !pos_dev || !sel_idx || !sel_cnt || !out || !ws) return RECSA_E_INVALID;
  if (!a16(q) || !a8(pos_dev) || !a4(sel_idx) || !a4(sel_cnt) || !a16(out) || !a16(ws))
    return RECSA_E_INVALID;
  if (!queries_fit(tree, T)) return RECSA_E_INVALID;
  const WsLayout w = ws_layout(*tree, Hq, static_cast<int64_t>(tree->B) * T);
  if (ws_bytes < static_cast<size_t>(w.total)) return RECSA_E_WORKSPACE;
  return hip_status(launch_attn(*tree, q, Hq, T, pos_dev, sel_idx, sel_cnt, out, ws, w, decode,
                                static_cast<hipStream_t>(stream)));
}

int recsa_attn_decode(const recsa_tree* tree, const void* q, int32_t Hq, const int64_t* pos_dev,
                      const int32_t* sel_idx, const int32_t* sel_cnt, float* out, void* ws,
                      size_t ws_bytes, void* stream) {
  return attn_common(tree, q, Hq, 1, pos_dev, sel_idx, sel_cnt, out, ws, ws_bytes, true, stream);
}

int recsa_attn_prefill(const recsa_tree* tree, const void* q, int32_t Hq, int32_t T,
                       const int64_t* pos_dev, const int32_t* sel_idx, const int32_t* sel_cnt,
                       float* out, void* ws, size_t ws_bytes, void* stream) {
  return attn_common(tree, q, Hq, T, pos_dev, sel_idx, sel_cnt, out, ws, ws_bytes, false, stream);
}

int recsa_decode(const recsa_tree* tree, const recsa_pooler* pooler, const void* k_new,
                 const void* v_new, const void* q, int32_t Hq, const int64_t* pos_dev,
                 int32_t* sel_idx, int32_t* sel_cnt, float* out, void* ws, size_t ws_bytes,
                 void* stream) {
  int why;
  if (!tree_ok(tree, &why)) return why;
  if (!pooler_ok(pooler, tree)) return RECSA_E_INVALID;
  if (!heads_ok(tree, Hq)) return RECSA_E_UNSUPPORTED;
  if (!k_new || !v_new || !q || !pos_dev || !sel_idx || !sel_cnt || !out || !ws)
    return RECSA_E_INVALID;
  if (!a16(k_new) || !a16(v_new) || !a16(q) || !a8(pos_dev) || !a4(sel_idx) || !a4(sel_cnt) ||
      !a16(out) || !a16(ws))
    return RECSA_E_INVALID;
  const WsLayout w = ws_layout(*tree, Hq, tree->B);
  if (ws_bytes < static_cast<size_t>(w.total)) return RECSA_E_WORKSPACE;
  const hipError_t e = launch_decode_fused(*tree, *pooler, k_new, v_new, q, Hq, pos_dev, sel_idx,
                                           sel_cnt, out, ws, w, static_cast<hipStream_t>(stream));
  if (e == hipErrorLaunchOutOfResources) return RECSA_E_UNSUPPORTED;
  return hip_status(e);
}

int recsa_decode_static(const recsa_tree* tree, const recsa_pooler* pooler, const void* k_new,
                        const void* v_new, const void* q, int32_t Hq, const int64_t* pos_dev,
                        int32_t* sel_idx, int32_t* sel_cnt, float* out, void* stream) {
  int why;
  if (!tree_ok(tree, &why)) return why;
  if (!pooler_ok(pooler, tree)) return RECSA_E_INVALID;
  if (!heads_ok(tree, Hq)) return RECSA_E_UNSUPPORTED;
  if (!k_new || !v_new || !q || !pos_dev || !sel_idx || !sel_cnt || !out) return RECSA_E_INVALID;
  if (!a16(k_new) || !a16(v_new) || !a16(q) || !a8(pos_dev) || !a4(sel_idx) || !a4(sel_cnt) ||
      !a16(out))
    return RECSA_E_INVALID;
  const WsLayout w = ws_layout(*tree, Hq, tree->B);
  if (w.total > static_cast<int64_t>(kStaticScratchBytes)) return RECSA_E_WORKSPACE;
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return RECSA_E_HIP;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the control block starts every call at zero (a call that timed out left
  // it in an undefined state)
  const int64_t n_ctl = (w.total - w.ctl_off) / 4;
  zero_words_kernel<<<static_cast<unsigned>((n_ctl + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + w.ctl_off), n_ctl);
  e = hipGetLastError();
  if (e != hipSuccess) return RECSA_E_HIP;
  e = launch_decode_fused(*tree, *pooler, k_new, v_new, q, Hq, pos_dev, sel_idx, sel_cnt, out, ws,
                          w, s);
  if (e == hipErrorLaunchOutOfResources) return RECSA_E_UNSUPPORTED;
  return hip_status(e);
}

// ---- pooler distillation losses

static bool distill_fits(const recsa_tree* t) {
  return distill_groups(t->L_cap) + static_cast<int64_t>(t->C) * t->k + 32 <= 16384;
}

size_t recsa_distill_workspace_bytes(const recsa_tree* tree, int32_t Hq, int64_t n_queries) {
  int why;
  if (!tree_ok(tree, &why) || !heads_ok(tree, Hq) || n_queries < 1 || !distill_fits(tree))
    return 0;
  return static_cast<size_t>(distill_ws_bytes(*tree, Hq, n_queries));
}

int recsa_distill_kl(const recsa_tree* tree, const void* q, int32_t Hq, int32_t T,
                     const int64_t* pos_dev, const int32_t* sel_idx, const int32_t* sel_cnt,
                     const float* importance, double theta, float* kl_out,
                     float* teacher_or_null, void* ws, size_t ws_bytes, void* stream) {
  int why;
  if (!tree_ok(tree, &why)) return why;
  if (!heads_ok(tree, Hq)) return RECSA_E_UNSUPPORTED;
  if (!q || T < 1 || !pos_dev || !sel_idx || !sel_cnt || !importance || !kl_out || !ws)
    return RECSA_E_INVALID;
  if (!a16(q) || !a8(pos_dev) || !a4(sel_idx) || !a4(sel_cnt) || !a16(importance) ||
      !a4(kl_out) || !a16(teacher_or_null) || !a16(ws))
    return RECSA_E_INVALID;
  if (!(theta > 1.0) || !queries_fit(tree, T)) return RECSA_E_INVALID;
  if (!distill_fits(tree)) return RECSA_E_UNSUPPORTED;
  if (ws_bytes < static_cast<size_t>(distill_ws_bytes(*tree, Hq, static_cast<int64_t>(tree->B) * T)))
    return RECSA_E_WORKSPACE;
  if (tree->n_levels < 2) return RECSA_OK;      // no level above the tokens: no term
  return hip_status(launch_distill_kl(*tree, q, Hq, T, pos_dev, sel_idx, sel_cnt, importance,
                                      theta, kl_out, teacher_or_null, ws,
                                      static_cast<hipStream_t>(stream)));
}

static bool shift_fits(const recsa_tree* t) {
  return (level_rows_host(t->L_cap, 1) + 15) / 16 <= 0x7FFFFFFF;
}

size_t recsa_shift_workspace_bytes(const recsa_tree* tree) {
  int why;
  if (!tree_ok(tree, &why) || !shift_fits(tree)) return 0;
  return static_cast<size_t>(shift_ws_bytes(*tree));
}

int recsa_shift_penalty(const recsa_tree* tree, const recsa_pooler* pooler, int64_t tok_end,
                        float* out, void* ws, size_t ws_bytes, void* stream) {
  int why;
  if (!tree_ok(tree, &why)) return why;
  if (!pooler_ok(pooler, tree) || !out || !ws || !a16(out) || !a16(ws)) return RECSA_E_INVALID;
  if (tok_end < 1 || tok_end > tree->L_cap) return RECSA_E_INVALID;
  if (!shift_fits(tree)) return RECSA_E_UNSUPPORTED;
  if (ws_bytes < static_cast<size_t>(shift_ws_bytes(*tree))) return RECSA_E_WORKSPACE;
  if (tree->n_levels < 2) return RECSA_OK;
  return hip_status(launch_shift_penalty(*tree, *pooler, tok_end, out, ws,
                                         static_cast<hipStream_t>(stream)));
}

// ---- gradient of the Eq. 6 terms with respect to the node keys

size_t recsa_distill_key_grad_workspace_bytes(const recsa_tree* tree, int32_t Hq,
                                              int64_t n_queries) {
  int why;
  if (!tree_ok(tree, &why) || !heads_ok(tree, Hq) || n_queries < 1) return 0;
  return static_cast<size_t>(kgrad_ws_bytes(*tree, Hq, n_queries));
}

int recsa_distill_key_grad(const recsa_tree* tree, const void* q, int32_t Hq, int32_t T,
                           const int64_t* pos_dev, const int32_t* sel_idx,
                           const int32_t* sel_cnt, const float* importance,
                           const float* teacher, const void* select_ws,
                           size_t select_ws_bytes, float* dK_out, void* ws, size_t ws_bytes,
                           void* stream) {
  int why;
  if (!tree_ok(tree, &why)) return why;
  if (!heads_ok(tree, Hq)) return RECSA_E_UNSUPPORTED;
  if (!q || T < 1 || !pos_dev || !sel_idx || !sel_cnt || !importance || !teacher ||
      !select_ws || !dK_out || !ws)
    return RECSA_E_INVALID;
  if (!a16(q) || !a8(pos_dev) || !a4(sel_idx) || !a4(sel_cnt) || !a16(importance) ||
      !a16(teacher) || !a16(select_ws) || !a16(dK_out) || !a16(ws))
    return RECSA_E_INVALID;
  if (!queries_fit(tree, T)) return RECSA_E_INVALID;
  const int64_t nq = static_cast<int64_t>(tree->B) * T;
  const WsLayout w = ws_layout(*tree, Hq, nq);
  if (select_ws_bytes < static_cast<size_t>(w.total) ||
      ws_bytes < static_cast<size_t>(kgrad_ws_bytes(*tree, Hq, nq)))
    return RECSA_E_WORKSPACE;
  if (tree->n_levels < 2) return RECSA_OK;
  const float* logits = reinterpret_cast<const float*>(static_cast<const char*>(select_ws) +
                                                       w.logits_off);
  return hip_status(launch_kgrad(*tree, q, Hq, T, pos_dev, sel_idx, sel_cnt, importance, teacher,
                                 logits, dK_out, ws, static_cast<hipStream_t>(stream)));
}

// ---- pooler backward

static bool grad_ok(const recsa_pooler_grad* g) {
  return g && g->w && g->W1 && g->b1 && g->W2 && g->tau && g->g && a16(g->w) && a16(g->W1) &&
         a16(g->b1) && a16(g->W2) && a4(g->tau) && a4(g->g);
}

size_t recsa_pooler_backward_workspace_bytes(const recsa_tree* tree, const recsa_pooler* pooler,
                                             int32_t level) {
  int why;
  if (!tree_ok(tree, &why) || !pooler_ok(pooler, tree) || !shift_fits(tree)) return 0;
  if (level < 1 || level >= tree->n_levels) return 0;
  return static_cast<size_t>(pool_bwd_ws_bytes(*tree, *pooler, level));
}

int recsa_pooler_backward(const recsa_tree* tree, const recsa_pooler* pooler, int32_t level,
                          int64_t tok_end, const float* dK, const float* shift_sums,
                          float shift_weight, const recsa_pooler_grad* grad, void* ws,
                          size_t ws_bytes, void* stream) {
  int why;
  if (!tree_ok(tree, &why)) return why;
  if (!pooler_ok(pooler, tree) || !grad_ok(grad) || !ws) return RECSA_E_INVALID;
  if (!a16(dK) || !a4(shift_sums) || !a16(ws)) return RECSA_E_INVALID;
  if (level < 1 || level >= tree->n_levels) return RECSA_E_INVALID;
  if (tok_end < 1 || tok_end > tree->L_cap || !isfinite(shift_weight)) return RECSA_E_INVALID;
  if (!shift_fits(tree)) return RECSA_E_UNSUPPORTED;
  if (ws_bytes < static_cast<size_t>(pool_bwd_ws_bytes(*tree, *pooler, level)))
    return RECSA_E_WORKSPACE;
  return hip_status(launch_pool_backward(*tree, *pooler, level, tok_end, dK, shift_sums,
                                         shift_weight, *grad, ws,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"
