/*
 * recsa.h -- C ABI of librecsa.so, the MI355X (gfx950) hot path of RecSA,
 * "Recursive Sparse Attention: Million-Token Length Extrapolation at
 * Logarithmic Cost" (arXiv 2611.07232).
 *
 * The pages (picx.dev summary, "Methodology") define the operation:
 *   - Tree Construction, Eq. 1: per layer and KV head, level 0 holds the
 *     exact token keys/values; C = 16 consecutive entries of a level form a
 *     parent whose key comes from a pooler and whose value is the mean of the
 *     children's values.
 *   - Pooler Distillation, Eq. 5: the pooler that makes a node key from its C
 *     children keys (one pooler per layer, shared by all levels: abstract).
 *   - Hierarchical Selection, Eq. 3: top-down, each level >= 1 keeps the
 *     current node plus the k-1 highest-scoring other candidates; the kept
 *     nodes' children form the next candidate list.
 *   - Key Theoretical Insight: each entry's RoPE position is its index in its
 *     level's candidate list, so every distance stays below C*k.
 *   - Unified Softmax, Eq. 4: one softmax over the exact level-0 candidates
 *     and the summaries of the unselected candidates of every level >= 1.
 *
 * Conventions shared by every call
 *   - All tensors are device memory owned by the caller.  The library never
 *     allocates, frees or synchronises; every call is ordered on `stream`
 *     (a hipStream_t passed as void*; NULL = the legacy default stream) and
 *     may be captured into a HIP graph.
 *   - Storage dtype (tree, q, k_new, v_new) is RECSA_F32 (float) or
 *     RECSA_BF16 (bfloat16 bits in uint16).  Arithmetic is float32; outputs
 *     are float32.
 *   - Query head h belongs to KV head h / (Hq / Hkv), with Hq / Hkv in
 *     {1, 2, 4} (other ratios return RECSA_E_UNSUPPORTED).  One selection is
 *     made per (query, KV head) and shared by its Hq/Hkv query heads.
 *   - q and the level-0 keys are given before RoPE: positions are assigned
 *     at query time from the candidate lists.
 *   - Logit of query head h and an entry at list position p (p = C*r + c) of
 *     a list whose last position is p_q = C*r_q + c_q:
 *         s = (q~ . k~) / sqrt(d),
 *         q~ = rnd(R(C*(r_q - r) + c_q) q_h),  k~ = rnd(R(c) K_entry),
 *     R = rotate-half RoPE (pairs (j, j+d/2), angle phi * theta^(-2j/d)),
 *     evaluated in float32 as (x*c - y*s, x*s + y*c) without fused
 *     multiply-add; rnd rounds to the storage dtype (nearest even).  In exact
 *     arithmetic this is q . R(p - p_q) K, RoPE at candidate-local positions.
 *   - Importance at a scored level (the pages leave it open) is the mean over
 *     the G query heads of the softmax of s over the non-current candidates;
 *     ties go to the smaller node index.
 *   - Alignment: arrays of float32 or bf16 values (tree levels, rope, q,
 *     k_new, v_new, outputs, importances, teacher distributions, gradients,
 *     pooler weights, workspaces) must be 16-byte aligned, since the kernels
 *     access them 16 bytes at a time; index arrays need their element's
 *     alignment, and so do the per-query KL output, one row of the shift
 *     penalty output and the two scalar gradients.  Every HIP or torch
 *     allocation, and every whole-row slice of one, qualifies.  Otherwise the
 *     call returns RECSA_E_INVALID.
 *   - Return value: RECSA_OK or a negative status.  Arguments are validated
 *     before anything is launched; on an error nothing is launched.
 *     RECSA_E_HIP reports a failed launch (hipGetLastError).
 */
#ifndef RECSA_H
#define RECSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RECSA_OK 0
#define RECSA_E_INVALID (-1)     /* null pointer, bad shape, range error      */
#define RECSA_E_UNSUPPORTED (-2) /* C != 16, d not 64/128, k > 512, dtype    */
#define RECSA_E_WORKSPACE (-3)   /* workspace smaller than required           */
#define RECSA_E_HIP (-4)         /* HIP launch error                          */

#define RECSA_F32 0
#define RECSA_BF16 1

#define RECSA_MAX_LEVELS 8

/* One layer's KV tree.
 * K[l], V[l]: level l rows, layout [B][Hkv][recsa_level_rows(L_cap, C, l)][d]
 *   in the storage dtype; level 0 is the ordinary KV cache (pre-RoPE keys).
 *   Only complete nodes are ever written: node i of level l covers tokens
 *   [i*C^l, (i+1)*C^l).
 * Kr[l]: optional -- every level NULL, or every level with rows set (a mix
 *   is RECSA_E_INVALID).  NULL: the tree is K and V only, and levels >= 1 add
 *   1/15 of the KV cache (picx.dev Practical Implications: under 7%); the
 *   kernels rotate each key row they read.  Set: a speed path that costs one
 *   more array of K's size (the cache grows to 1.5x K+V), laid out like K,
 *   whose row i holds the key half of the split RoPE, rnd(R(i mod C)
 *   K[l][i]) (see the logit below), which depends on the row alone; the
 *   library writes it for every row it writes (nodes built or appended, the
 *   appended token) and, in recsa_build_tree, for the level-0 rows of the
 *   given token range, and selection and attention then read keys from it.
 *   Both forms give identical results (the in-kernel rotation uses the same
 *   float32 rotation and rounding).
 * n_levels: levels allocated, >= recsa_levels_needed(L_cap, C, k) (so the
 *   list of the top level has at most k nodes for every position < L_cap);
 *   more levels do not change any result.
 * rope: float32 table [C*k][d/2][2] of (cos, sin), filled by recsa_init_rope.
 * Level 0 (K[0], V[0] and Kr[0] if kept) may be page-locked host memory that the device
 * can address (hipHostMalloc; pass the address hipHostGetDevicePointer
 * returns): every call then reads and writes the level-0 rows it needs in
 * place over PCIe, with identical results, while levels >= 1 (1/15 of the
 * cache) stay in device memory (picx.dev Efficiency Results, KV offloading;
 * Practical Implications, bounded GPU memory).
 */
typedef struct recsa_tree {
  int32_t dtype;
  int32_t B;
  int32_t Hkv;
  int32_t d;
  int32_t C;
  int32_t k;
  int32_t n_levels;
  int32_t reserved;
  int64_t L_cap;
  void* K[RECSA_MAX_LEVELS];
  void* V[RECSA_MAX_LEVELS];
  void* Kr[RECSA_MAX_LEVELS];
  const float* rope;
} recsa_tree;

/* The pooler of Eq. 5, float32 device arrays, one per layer:
 *   mu = mean_c x_c;  sigma = sqrt(mean_{c,j} (x_cj - mu_j)^2 + eps);
 *   rho = sqrt(mean_j mu_j^2 + eps);
 *   alpha = softmax_c(tau * w.(x_c - mu) / sigma);  p = sum_c alpha_c x_c;
 *   m = W2 SiLU(W1 [mu/rho ; (p - mu)/sigma] + b1);
 *   K = mu + g (p - mu) + sigma m.
 * w: [d]; W1: [hidden][2d] row-major; b1: [hidden]; W2: [d][hidden].
 * hidden must be a multiple of 16 and at most 256. */
typedef struct recsa_pooler {
  int32_t d;
  int32_t hidden;
  float tau;
  float g;
  float eps;
  int32_t reserved;
  const float* w;
  const float* W1;
  const float* b1;
  const float* W2;
} recsa_pooler;

/* Human-readable name of a status code (static string, never NULL). */
const char* recsa_status_string(int status);

/* Rows allocated at `level` for capacity L_cap: floor(L_cap / C^level). */
int64_t recsa_level_rows(int64_t L_cap, int32_t C, int32_t level);

/* Smallest level count whose top list [0 .. floor(t / C^(n-1))] has at most
 * k nodes for every t < L_cap (the walk starts there; Eq. 3 first line). */
int32_t recsa_levels_needed(int64_t L_cap, int32_t C, int32_t k);

/* Fill the RoPE table `table` [n_pos][d/2][2] (device, float32) with
 * cos/sin(phi * theta^(-2j/d)), evaluated in double and rounded once.
 * n_pos must be C*k for use in a recsa_tree. */
int recsa_init_rope(float* table, int32_t d, int32_t n_pos, double theta, void* stream);

/* Workspace bytes recsa_select and recsa_attn_* need for n_queries = B*T
 * queries with Hq query heads (logits of every scored candidate, selection
 * bitmaps and attention partials).  0 on invalid arguments. */
size_t recsa_workspace_bytes(const recsa_tree* tree, int32_t Hq, int64_t n_queries);

/* Tree Construction (Eq. 1, Eq. 5): write the rotated keys Kr[0] of the
 * level-0 rows [tok_begin, tok_end) (when the tree keeps Kr), then
 * (re)compute every complete node, at every level >= 1, whose last token lies
 * in [tok_begin, tok_end), with its rotated key.  Level-0 rows [0, tok_end) must already be written.  Nodes are
 * computed level by level, each from the stored (rounded) children.
 * 0 <= tok_begin <= tok_end <= L_cap. */
int recsa_build_tree(const recsa_tree* tree, const recsa_pooler* pooler,
                     int64_t tok_begin, int64_t tok_end, void* stream);

/* Decode append: for each sequence b write k_new/v_new [B][Hkv][d] as level-0
 * row t = pos_dev[b] (device int64 [B]), with its rotated key, and complete
 * every node whose last token is t (levels l with (t+1) mod C^l == 0).  Precondition (device side,
 * not checked): 0 <= t < L_cap and rows [0, t) are in the tree. */
int recsa_append_decode(const recsa_tree* tree, const recsa_pooler* pooler,
                        const void* k_new, const void* v_new,
                        const int64_t* pos_dev, void* stream);

/* Hierarchical Selection (Eq. 3) for T queries per sequence.
 * q: [B][T][Hq][d] storage dtype; pos_dev: [B][T] device int64, each query's
 *   token position t (the query attends over tokens [0, t]; row t and every
 *   complete node over [0, t) must be in the tree).
 * sel_idx: [B][T][Hkv][n_levels-1][k] int32: slot l-1 holds S^(l) in ascending
 *   node order (the current node last), -1 padded.
 * sel_cnt: [B][T][Hkv][n_levels-1] int32 = |S^(l)|.
 * importance_or_null: optional [B][T][Hkv][n_levels-1][C*k] float32; entry p
 *   is the importance of the candidate at list position p (0 where unscored).
 * ws: workspace of at least recsa_workspace_bytes(tree, Hq, B*T) bytes; it
 *   keeps the logits that recsa_attn_* reuse for the unselected summaries, so
 *   pass the same ws, untouched, to the attention call of the same queries. */
int recsa_select(const recsa_tree* tree, const void* q, int32_t Hq, int32_t T,
                 const int64_t* pos_dev, int32_t* sel_idx, int32_t* sel_cnt,
                 float* importance_or_null, void* ws, size_t ws_bytes,
                 void* stream);

/* Unified Softmax (Eq. 4) for one decode query per sequence: q [B][Hq][d],
 * pos_dev [B], the selection and ws of recsa_select (T = 1); out [B][Hq][d]
 * float32.  The launch shape depends only on the tree's static sizes. */
int recsa_attn_decode(const recsa_tree* tree, const void* q, int32_t Hq,
                      const int64_t* pos_dev, const int32_t* sel_idx,
                      const int32_t* sel_cnt, float* out, void* ws,
                      size_t ws_bytes, void* stream);

/* Unified Softmax (Eq. 4) for T queries per sequence (a causal prefill
 * chunk): q [B][T][Hq][d], pos_dev [B][T], selection and ws of recsa_select;
 * out [B][T][Hq][d] float32. */
int recsa_attn_prefill(const recsa_tree* tree, const void* q, int32_t Hq,
                       int32_t T, const int64_t* pos_dev,
                       const int32_t* sel_idx, const int32_t* sel_cnt,
                       float* out, void* ws, size_t ws_bytes, void* stream);

/* One decode step in a single launch: recsa_append_decode, recsa_select (T = 1)
 * and recsa_attn_decode with the same arguments and results, for when the
 * caller wants the lowest latency.  The (sequence, KV head) pairs are each
 * served by a group of workgroups that must all be resident at once; the
 * call returns RECSA_E_UNSUPPORTED when B*Hkv groups cannot be.
 * ws: recsa_workspace_bytes(tree, Hq, B) bytes whose control block (the last
 * B*Hkv*2112 bytes: 528 32-bit words per (sequence, KV head)) is zero before
 * the first call -- a zero-filled workspace satisfies this -- and is left
 * zero by every call that succeeds.  Should a group ever wait longer than
 * its bounded spin, word 1 of its block (the error word) is set to nonzero
 * and its output is NaN; the rest of the block is then in an undefined
 * state, and the caller must zero the whole control block before the next
 * call with this ws.  Calls sharing one ws must not overlap.
 * Precondition: the launch sizes each group's workgroups to fit the device
 * with room to spare, assuming no other kernel occupies it; a kernel running
 * concurrently on another stream can keep a group's workgroups from being
 * placed, which then shows as the timeout above (NaN, error word set),
 * never as a silently wrong result. */
int recsa_decode(const recsa_tree* tree, const recsa_pooler* pooler,
                 const void* k_new, const void* v_new, const void* q, int32_t Hq,
                 const int64_t* pos_dev, int32_t* sel_idx, int32_t* sel_cnt,
                 float* out, void* ws, size_t ws_bytes, void* stream);

/* recsa_decode without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and launch as
 * recsa_decode, except that the workspace is the library's own device array
 * of 32 MiB (one per device, set up on the first call on that device and
 * held until the process ends); the call allocates nothing.  Each call first
 * zeroes the array's control block with a kernel, so no state carries over
 * from an earlier call, including one that timed out.  Configurations whose
 * recsa_workspace_bytes(tree, Hq, B) exceeds 32 MiB return
 * RECSA_E_WORKSPACE (for example 8 sequences x 8 KV heads at G = 4, k = 256
 * and 5 levels need 25 MiB; 16 x 8 do not fit).  Every call on one device
 * shares that device's array: calls that overlap on one device (two streams,
 * two threads) race and give undefined results.  A timed-out wait makes the
 * output NaN, as in recsa_decode. */
int recsa_decode_static(const recsa_tree* tree, const recsa_pooler* pooler,
                        const void* k_new, const void* v_new, const void* q, int32_t Hq,
                        const int64_t* pos_dev, int32_t* sel_idx, int32_t* sel_cnt,
                        float* out, void* stream);

/* ---- Pooler distillation losses (picx.dev Pooler Distillation, Eq. 6 and
 * Eq. 7).  Readings of their operands: the teacher is the dense causal
 * attention of the same G query heads at position t over the level-0 tokens
 * [0, t], with RoPE at the true positions (angle (tau - t) theta^(-2j/d)),
 * scale 1/sqrt(d); y_t^(l) is its head-mean mass under each non-current
 * candidate of A_t^(l), renormalised over those candidates (the support of
 * pi); pi_t^(l) is the importance recsa_select reports; only scored levels
 * (|A| > k) have a term; the shift penalty of level l averages over every
 * complete level-l node of every sequence and KV head. */

/* Workspace bytes of recsa_distill_kl for n_queries = B*T queries with Hq
 * query heads: the RoPE table of the absolute positions [0, L_cap), float32
 * [L_cap][d/2][2]; every level-0 key rotated at its position and split into
 * two bf16 halves, [B][Hkv][L_cap][2][d]; then the teacher's per-group
 * log-sum-exps, float32 [n_queries][Hkv][ceil(L_cap/16)][Hq/Hkv].  0 on
 * invalid arguments. */
size_t recsa_distill_workspace_bytes(const recsa_tree* tree, int32_t Hq,
                                     int64_t n_queries);

/* Eq. 6 terms of T queries per sequence.  q, pos_dev, sel_idx and sel_cnt as
 * in recsa_select (pos_dev [B][T] device int64); importance: the importance
 * output of recsa_select for the same queries (required).  theta: the RoPE
 * base (> 1).  Level-0 rows [0, t] of each query must be in the tree.
 * kl_out: [B][T][Hkv][n_levels-1] float32: slot l-1 holds KL(y || pi) of
 * level l when it is scored, else 0; a zero importance under a positive
 * teacher mass gives +inf.
 * teacher_or_null: optional [B][T][Hkv][n_levels-1][C*k] float32, laid out
 * like the importance: entry p is y of the candidate at list position p (0
 * for the current node, past the list and at unscored levels).  With the
 * importance and the logits it gives d KL / d logit in closed form.  Arithmetic is float32 (teacher logits on the
 * float32 matrix cores).  ws: recsa_distill_workspace_bytes(tree, Hq, B*T)
 * bytes of device memory, overwritten.  RECSA_E_UNSUPPORTED when
 * ceil(L_cap/16) + C*k exceeds 16352 (the masses of one query are kept on
 * chip). */
int recsa_distill_kl(const recsa_tree* tree, const void* q, int32_t Hq, int32_t T,
                     const int64_t* pos_dev, const int32_t* sel_idx,
                     const int32_t* sel_cnt, const float* importance, double theta,
                     float* kl_out, float* teacher_or_null, void* ws,
                     size_t ws_bytes, void* stream);

/* Workspace bytes of recsa_shift_penalty: one partial row of d+1 floats per
 * 16 nodes of every level >= 1, (sequence, KV head).  0 on invalid
 * arguments. */
size_t recsa_shift_workspace_bytes(const recsa_tree* tree);

/* Eq. 7 for every level l >= 1 over its complete nodes among the tokens
 * [0, tok_end) of every sequence and KV head (M_l nodes), each node's pooler
 * parts recomputed in float32 from its stored children.  out:
 * [n_levels-1][d+2] float32; slot l-1 holds the sum over those nodes of
 * sigma*m (d values), the sum of ||mu||^2, then the penalty
 * ||sum sigma m||^2 / (M_l * sum ||mu||^2) (0 where the level has no complete
 * node).  The sums are taken in a fixed order: repeated calls give identical
 * bits.  ws: recsa_shift_workspace_bytes(tree) bytes, overwritten.
 * 0 < tok_end <= L_cap. */
int recsa_shift_penalty(const recsa_tree* tree, const recsa_pooler* pooler,
                        int64_t tok_end, float* out, void* ws, size_t ws_bytes,
                        void* stream);

/* Workspace bytes of recsa_distill_key_grad: each query head's softmax
 * figures at each level, four float32 per [B*T][Hkv][n_levels-1][Hq/Hkv]
 * (rounded up to 256 bytes), then float32 partial sums per chunk of 2048
 * queries, [B][Hkv][ceil(rows of level 1 / C)][ceil(T/2048)][C][d].  0 on
 * invalid arguments. */
size_t recsa_distill_key_grad_workspace_bytes(const recsa_tree* tree, int32_t Hq,
                                              int64_t n_queries);

/* Gradient of the Eq. 6 terms of T queries per sequence, sum over queries,
 * KV heads and scored levels of KL(y || pi), with respect to every stored
 * node key (picx.dev Pooler Distillation, Eq. 6).  With P_h the softmax of
 * head h's logits over a level's non-current candidates, pi = mean_h P_h and
 * r = y / pi: d KL / d s_h,e = -(P_h,e / G) (r_e - sum_f r_f P_h,f); each logit
 * s_h,e = q~_h . k~_e / sqrt(d) (the split candidate-local RoPE of
 * recsa_select, operand roundings taken as the identity) adds
 * R(c_e)^T q~_h / sqrt(d) times that to its key.  This is the dK that
 * recsa_pooler_backward takes.
 * q, pos_dev, sel_idx, sel_cnt, importance: as given to and returned by
 * recsa_select; select_ws: that call's workspace (its logits are read);
 * teacher: the teacher distributions of recsa_distill_kl for the same queries.
 * dK_out: float32 device array, the levels 1 .. n_levels-1 one after another,
 * level l as [B][Hkv][recsa_level_rows(L_cap, C, l)][d]; every element is
 * written (0 where no query scores the node).  Each element is summed over
 * the queries in order: identical bits on every call.  ws:
 * recsa_distill_key_grad_workspace_bytes(tree, Hq, B*T) bytes. */
int recsa_distill_key_grad(const recsa_tree* tree, const void* q, int32_t Hq, int32_t T,
                           const int64_t* pos_dev, const int32_t* sel_idx,
                           const int32_t* sel_cnt, const float* importance,
                           const float* teacher, const void* select_ws,
                           size_t select_ws_bytes, float* dK_out, void* ws,
                           size_t ws_bytes, void* stream);

/* Gradients of the pooler parameters, float32 device arrays shaped like the
 * fields of recsa_pooler (tau and g: one float each). */
typedef struct recsa_pooler_grad {
  float* w;    /* [d] */
  float* W1;   /* [hidden][2d] */
  float* b1;   /* [hidden] */
  float* W2;   /* [d][hidden] */
  float* tau;  /* [1] */
  float* g;    /* [1] */
} recsa_pooler_grad;

/* Workspace bytes of recsa_pooler_backward at `level`: one row of
 * 3d + 2*hidden floats per node slot, d+2 floats per 16 nodes, and one
 * float64 partial of every gradient element per 512 node slots.  0 on
 * invalid arguments. */
size_t recsa_pooler_backward_workspace_bytes(const recsa_tree* tree,
                                             const recsa_pooler* pooler,
                                             int32_t level);

/* Pooler backward (picx.dev Pooler Distillation, Eq. 5; Training Stages,
 * stage 1): gradients of
 *     L = sum_i dK_i . K_i + shift_weight * penalty_level
 * with respect to every pooler parameter, over the complete nodes i of
 * `level` (>= 1) among the tokens [0, tok_end) of every sequence and KV
 * head.  Each node's key K_i is recomputed in float32 from its stored
 * children, which are inputs (no gradient flows into lower levels); the
 * rounding of the stored key is taken as the identity.
 * dK: [B][Hkv][recsa_level_rows(L_cap, C, level)][d] float32 device array
 *   (rows of nodes beyond the range are not read), or NULL for zero.
 * shift_sums: the level's row of recsa_shift_penalty output for the same
 *   tok_end (sum of sigma*m [d], sum of ||mu||^2, penalty), or NULL for no
 *   penalty term; its gradient reaches the parameters through m only.
 * grad: overwritten (not accumulated); every element is a float64 sum in
 *   node order, so repeated calls give identical bits.
 * ws: recsa_pooler_backward_workspace_bytes bytes, overwritten.
 * 0 < tok_end <= L_cap; 1 <= level < n_levels. */
int recsa_pooler_backward(const recsa_tree* tree, const recsa_pooler* pooler,
                          int32_t level, int64_t tok_end, const float* dK,
                          const float* shift_sums, float shift_weight,
                          const recsa_pooler_grad* grad, void* ws,
                          size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RECSA_H */
