"""Plain CPU oracle for RecSA (Recursive Sparse Attention).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only the tests, the smoke check of the graft entry point and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP path.

Source: "Recursive Sparse Attention: Million-Token Length Extrapolation at
Logarithmic Cost" (Wang, Yang, Zhang, Zhang; arXiv 2611.07232), as summarised
on the picx.dev page ("Methodology": Tree Construction Eq. 1, Hierarchical
Selection Eq. 3, Unified Softmax Eq. 4, Pooler Distillation Eq. 5) and the
abstract on the paper-reader page.

Everything is NumPy in float64, on one KV head at a time, with loops where the
pages state a loop.  Inputs are the stored (storage-dtype) values lifted
exactly to float64.  Rounding happens only where stated:

* node keys and values are rounded to the storage dtype when stored;
* the two operands of every logit are rounded to the storage dtype after a
  float32 rotation (the "split" form of candidate-local RoPE).  That rounding
  decides a quantised code, so it is taken in the float32 precision the
  kernels use, with the operation order written out in ``rotate_f32``.

Readings of points the pages leave open:
  current node a_t^(l) = floor(t / C^l); the walk starts at the first level
  whose list [0..a] has at most k nodes; candidate lists are concatenated in
  ascending node order and the query sits at the last position; importance is
  the head-mean of the softmax over the non-current candidates; ties go to the
  smaller node index; rotate-half RoPE with a caller-given base; logit scale
  1/sqrt(d); sigma and rho are scalars with eps inside the square roots; the
  pooler's hidden width is free (h = d in the workloads); one pooler serves
  every level and every KV head of a layer.

Parity of the pooler's absolute outputs for random weights is pinned only by
invariants and special cases (see the pin tests); the pages print no worked
numeric example of it.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Pooler", "round_bf16", "rnd", "rope_table", "rotate_f32", "rotate_exact",
    "pool_keys", "mean_values", "level_sizes", "n_levels_for", "build_tree",
    "append_token", "walk", "attend", "decode_reference", "LevelTrace",
    "WalkTrace",
]

# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_SUB_STEP = 2.0 ** -133


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (7 stored) and float32's exponent range.
    Returned as float64 (exactly representable)."""
    orig = np.array(x, dtype=np.float64, copy=True)
    u = orig.copy().view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u += np.uint64((1 << 44) - 1) + lsb
    u &= ~np.uint64((1 << 45) - 1)
    out = u.view(np.float64)
    tiny = np.abs(orig) < _BF16_MIN_NORMAL
    if np.any(tiny):
        # subnormal bfloat16 range: fixed spacing 2^-133, ties to even
        out[tiny] = np.round(orig[tiny] / _BF16_SUB_STEP) * _BF16_SUB_STEP
    return out


def rnd(x, dtype: str):
    """Round to the storage dtype ('bf16' or 'f32'), returned as float64."""
    if dtype == "bf16":
        return round_bf16(np.asarray(x, dtype=np.float64))
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# RoPE (candidate-local positions; picx.dev "Key Theoretical Insight" and
# "Summary": each entry's position is its index in its level's list)
# --------------------------------------------------------------------------

def rope_table(d: int, n_pos: int, theta: float):
    """cos/sin of phi * theta^(-2j/d) for phi in [0, n_pos), j in [0, d/2).

    Computed in float64 and rounded once to float32 (the table precision)."""
    j = np.arange(d // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), (-2.0 * j) / d)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rotate_f32(v, cos_row, sin_row):
    """Rotate-half RoPE evaluated in float32 with a fixed operation order.

    Pair (j, j + d/2) = (x, y) becomes (x*c - y*s, x*s + y*c); every product
    and every sum is one correctly rounded float32 operation (no fused
    multiply-add).  Returns float32."""
    v = np.asarray(v, dtype=np.float32)
    h = v.shape[-1] // 2
    x, y = v[..., :h], v[..., h:]
    c = np.asarray(cos_row, dtype=np.float32)
    s = np.asarray(sin_row, dtype=np.float32)
    first = (x * c) - (y * s)
    second = (x * s) + (y * c)
    return np.concatenate([first, second], axis=-1)


def rotate_exact(v, pos, theta: float):
    """Rotate-half RoPE at (possibly fractional-free integer) position ``pos``
    in float64 with float64 trigonometry; no rounding.  ``pos`` broadcasts
    against the leading axes of ``v``."""
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    h = d // 2
    j = np.arange(h, dtype=np.float64)
    inv_freq = np.power(float(theta), (-2.0 * j) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x, y = v[..., :h], v[..., h:]
    return np.concatenate([x * c - y * s, x * s + y * c], axis=-1)


# --------------------------------------------------------------------------
# Tree construction (picx.dev "Tree Construction", Eq. 1; pooler Eq. 5)
# --------------------------------------------------------------------------

@dataclass
class Pooler:
    """Parameters of the pooler of Eq. 5 (one per layer, shared by all levels).

    w: [d]; tau, g: scalars; W1: [h, 2d]; b1: [h]; W2: [d, h]; eps: added
    inside the square roots of sigma and rho."""
    w: np.ndarray
    tau: float
    g: float
    W1: np.ndarray
    b1: np.ndarray
    W2: np.ndarray
    eps: float = 1e-6

    def as64(self) -> "Pooler":
        return Pooler(np.asarray(self.w, np.float64), float(self.tau),
                      float(self.g), np.asarray(self.W1, np.float64),
                      np.asarray(self.b1, np.float64),
                      np.asarray(self.W2, np.float64), float(self.eps))


def _silu(z):
    return z / (1.0 + np.exp(-z))


def pool_parts(X, P: Pooler):
    """The parts of Eq. 5 for a batch of nodes.

    X: [N, C, d] children keys (float64).  Returns (mu [N, d], sigma [N],
    p [N, d], m [N, d]):
        mu    = mean of the children
        sigma = sqrt(mean over children and dims of (x - mu)^2 + eps)
        rho   = sqrt(mean over dims of mu^2 + eps)
        alpha = softmax over children of tau * w.(x_c - mu) / sigma
        p     = sum_c alpha_c x_c
        m     = W2 SiLU(W1 [mu/rho ; (p - mu)/sigma] + b1)
    """
    P = P.as64()
    X = np.asarray(X, dtype=np.float64)
    mu = X.mean(axis=1)                                     # [N, d]
    dev = X - mu[:, None, :]                                 # [N, C, d]
    sigma = np.sqrt((dev * dev).mean(axis=(1, 2)) + P.eps)   # [N]
    rho = np.sqrt((mu * mu).mean(axis=1) + P.eps)            # [N]
    logits = P.tau * (dev @ P.w) / sigma[:, None]            # [N, C]
    logits = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    alpha = e / e.sum(axis=1, keepdims=True)                 # [N, C]
    p = np.einsum("nc,ncd->nd", alpha, X)                    # [N, d]
    feat = np.concatenate([mu / rho[:, None], (p - mu) / sigma[:, None]], axis=1)
    hidden = _silu(feat @ P.W1.T + P.b1)                     # [N, h]
    m = hidden @ P.W2.T                                      # [N, d]
    return mu, sigma, p, m


def pool_keys(X, P: Pooler):
    """Eq. 5 node keys (unrounded) for a batch of nodes, X: [N, C, d]:
    K = mu + g (p - mu) + sigma m, with the parts of ``pool_parts``."""
    mu, sigma, p, m = pool_parts(X, P)
    return mu + float(P.g) * (p - mu) + sigma[:, None] * m


def mean_values(X):
    """Eq. 1 value of a node: the plain mean of its C children. X: [N, C, d]."""
    return np.asarray(X, dtype=np.float64).mean(axis=1)


def level_sizes(n_tokens: int, C: int, n_levels: int):
    """Number of complete nodes per level: N_0 = n_tokens, N_l = floor(N_{l-1}/C)."""
    sizes = [int(n_tokens)]
    for _ in range(1, n_levels):
        sizes.append(sizes[-1] // C)
    return sizes


def n_levels_for(t_max: int, C: int, k: int) -> int:
    """Smallest number of levels D such that the top list [0 .. floor(t/C^(D-1))]
    has at most k nodes for every query position t <= t_max."""
    D = 1
    while (t_max // C ** (D - 1)) + 1 > k:
        D += 1
    return D


def build_tree(K0, V0, C: int, n_levels: int, P: Pooler, dtype: str):
    """Build levels 1..n_levels-1 over the stored level-0 rows K0, V0 [N0, d].

    Only complete nodes exist.  Each level reads the *stored* (rounded)
    values of the level below.  Returns lists K[l], V[l] of float64 arrays."""
    K = [rnd(K0, dtype)]
    V = [rnd(V0, dtype)]
    sizes = level_sizes(K[0].shape[0], C, n_levels)
    d = K[0].shape[1]
    for lvl in range(1, n_levels):
        n = sizes[lvl]
        kc = K[lvl - 1][: n * C].reshape(n, C, d)
        vc = V[lvl - 1][: n * C].reshape(n, C, d)
        K.append(rnd(pool_keys(kc, P), dtype) if n else np.zeros((0, d)))
        V.append(rnd(mean_values(vc), dtype) if n else np.zeros((0, d)))
    return K, V


def append_token(K, V, k_new, v_new, C: int, P: Pooler, dtype: str):
    """Append token t = len(K[0]) and complete every node whose last token is t.

    Returns new lists (inputs are not modified)."""
    K = [x.copy() for x in K]
    V = [x.copy() for x in V]
    d = K[0].shape[1]
    K[0] = np.concatenate([K[0], rnd(np.asarray(k_new).reshape(1, d), dtype)])
    V[0] = np.concatenate([V[0], rnd(np.asarray(v_new).reshape(1, d), dtype)])
    t = K[0].shape[0] - 1
    for lvl in range(1, len(K)):
        span = C ** lvl
        if (t + 1) % span != 0:
            break
        i = (t + 1) // span - 1
        kc = K[lvl - 1][i * C:(i + 1) * C].reshape(1, C, d)
        vc = V[lvl - 1][i * C:(i + 1) * C].reshape(1, C, d)
        assert K[lvl].shape[0] == i
        K[lvl] = np.concatenate([K[lvl], rnd(pool_keys(kc, P), dtype)])
        V[lvl] = np.concatenate([V[lvl], rnd(mean_values(vc), dtype)])
    return K, V


# --------------------------------------------------------------------------
# Hierarchical selection (picx.dev "Hierarchical Selection", Eq. 3) and the
# unified softmax (Eq. 4)
# --------------------------------------------------------------------------

@dataclass
class LevelTrace:
    level: int
    A: np.ndarray            # candidate node indices in list order (ascending)
    S: np.ndarray            # selected node indices, ascending
    scored: bool             # False when |A| <= k (everything selected)
    logits: np.ndarray | None = None       # [G, |A|-1] for the non-current entries
    importance: np.ndarray | None = None   # [|A|-1]
    S_own: np.ndarray | None = None        # the walk's own top-k choice (== S unless
                                           # a ``choose`` hook substituted another)


@dataclass
class WalkTrace:
    t: int
    levels: dict = field(default_factory=dict)   # level -> LevelTrace (levels >= 1)
    A0: np.ndarray | None = None                  # level-0 candidates (tokens)
    logits0: np.ndarray | None = None             # [G, |A0|]
    entries: list = field(default_factory=list)   # [(level, node)] of E_t
    entry_logits: np.ndarray | None = None        # [G, |E|]


def _operands_logits(qG, keys, pos_e, p_q, C, cos, sin, dtype, exact, theta):
    """Logits s[h, e] of the G query heads against ``keys`` sitting at list
    positions ``pos_e``, with the query at list position ``p_q``.

    Split form (exact == False): with p = C*r + c,
        q~ = rnd(R(C*(r_q - r_e) + c_q) q),   k~ = rnd(R(c_e) k),
    rotation in float32 (``rotate_f32``), rnd to the storage dtype, then the
    dot product in float64 and the 1/sqrt(d) scale.  In exact arithmetic this
    is q . R(p_e - p_q) k, i.e. RoPE at the candidate-local positions.
    Exact mode rotates q by p_q and k by p_e in float64 with no rounding."""
    qG = np.asarray(qG, dtype=np.float64)
    G, d = qG.shape
    pos_e = np.asarray(pos_e, dtype=np.int64)
    if exact:
        qr = rotate_exact(qG, p_q, theta)                    # [G, d]
        kr = rotate_exact(keys, pos_e, theta)                # [n, d]
        return (qr @ kr.T) / math.sqrt(d)
    r_q, c_q = divmod(int(p_q), C)
    r_e, c_e = pos_e // C, pos_e % C
    kt = rnd(rotate_f32(keys, cos[c_e], sin[c_e]).astype(np.float64), dtype)
    out = np.empty((G, len(pos_e)))
    for r in np.unique(r_e):
        sel = np.nonzero(r_e == r)[0]
        phi = C * (r_q - int(r)) + c_q
        qt = rnd(rotate_f32(qG, cos[phi], sin[phi]).astype(np.float64), dtype)
        out[:, sel] = qt @ kt[sel].T
    return out / math.sqrt(d)


def _children(S, a_below, C):
    """Next candidate list: concat over i in S (ascending) of
    [C*i, ..., min(C*i + C - 1, a_below)]  (Eq. 3, third line)."""
    out = []
    for i in sorted(int(x) for x in S):
        hi = min(C * i + C - 1, a_below)
        out.extend(range(C * i, hi + 1))
    return np.asarray(out, dtype=np.int64)


def _topk_lowest_index(I, nodes, m):
    """Indices (into ``nodes``) of the m largest importances; ties go to the
    smaller node index."""
    order = sorted(range(len(I)), key=lambda i: (-I[i], int(nodes[i])))
    return order[:m]


def walk(qG, t: int, K, C: int, k: int, cos=None, sin=None, dtype="f32",
         exact=False, theta=1e6, choose=None):
    """Top-down selection for one query at position t against one KV head's
    tree K (list of per-level key arrays; K[0] must hold rows 0..t).

    qG: [G, d] query heads sharing this KV head.  Returns a WalkTrace with the
    per-level lists A, selections S, logits and importances, the level-0 list
    and the entry set E_t of Eq. 4 with one logit per head and entry.

    choose: optional hook ``choose(level, others, I, S) -> S'`` called at
    every scored level with the non-current candidates, their importances and
    the walk's own selection; the walk continues with the returned set (a
    caller comparing against another implementation uses it to follow that
    implementation's choice at an accepted near-tie, so that one flipped
    near-tie does not change every list below it)."""
    qG = np.asarray(qG, dtype=np.float64)
    G, d = qG.shape
    n_levels = len(K)
    top = n_levels - 1
    a = [t // C ** lvl for lvl in range(n_levels)]
    tr = WalkTrace(t=t)
    A = np.arange(a[top] + 1, dtype=np.int64)
    if len(A) > k:
        raise ValueError("top level has more than k nodes; add a level")
    entries, ent_logits = [], []
    for lvl in range(top, 0, -1):
        cur = a[lvl]
        assert A[-1] == cur
        if len(A) <= k:
            S = A.copy()
            tr.levels[lvl] = LevelTrace(lvl, A, S, False)
        else:
            others = A[:-1]
            p_q = len(A) - 1
            s = _operands_logits(qG, K[lvl][others], np.arange(len(others)),
                                 p_q, C, cos, sin, dtype, exact, theta)
            # importance: head-mean of the softmax over the non-current nodes
            z = s - s.max(axis=1, keepdims=True)
            pi = np.exp(z)
            pi = pi / pi.sum(axis=1, keepdims=True)
            I = pi.mean(axis=0)
            keep = _topk_lowest_index(I, others, k - 1)
            S = np.sort(np.concatenate([others[keep], [cur]]))
            S_own = S
            if choose is not None:
                S = np.sort(np.asarray(choose(lvl, others, I, S), dtype=np.int64))
            tr.levels[lvl] = LevelTrace(lvl, A, S, True, s, I, S_own)
            chosen = set(int(x) for x in S)
            for i, node in enumerate(others):
                if int(node) not in chosen:
                    entries.append((lvl, int(node)))
                    ent_logits.append(s[:, i])
        A = _children(S, a[lvl - 1], C)
    # level 0: every candidate is an exact token, the query itself last
    assert A[-1] == t
    p_q = len(A) - 1
    s0 = _operands_logits(qG, K[0][A], np.arange(len(A)), p_q, C, cos, sin,
                          dtype, exact, theta)
    tr.A0, tr.logits0 = A, s0
    tok = [(0, int(x)) for x in A]
    tr.entries = tok + entries
    tr.entry_logits = np.concatenate(
        [s0] + ([np.stack(ent_logits, axis=1)] if ent_logits else []), axis=1)
    return tr


def attend(tr: WalkTrace, V):
    """Eq. 4: o_h = sum_e exp(s_he) V_e / sum_e exp(s_he) over E_t, float64.
    V: list of per-level value arrays.  Returns [G, d]."""
    rows = np.stack([V[lvl][node] for lvl, node in tr.entries])   # [E, d]
    s = tr.entry_logits                                            # [G, E]
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w @ rows) / w.sum(axis=1, keepdims=True)


def decode_reference(qG, t, K, V, C, k, cos, sin, dtype, exact=False, theta=1e6,
                     choose=None):
    """Walk plus attention for one query on one KV head."""
    tr = walk(qG, t, K, C, k, cos, sin, dtype, exact, theta, choose)
    return attend(tr, V), tr


# --------------------------------------------------------------------------
# Pooler distillation losses (picx.dev "Pooler Distillation", Eq. 6 and
# Eq. 7).  Readings (the pages give the formulas, not their operands):
#  * the teacher is the dense causal attention of the same G query heads at
#    position t over tokens 0..t, standard RoPE at the true positions,
#    softmax over s[h, tau] = q_h . R(tau - t) k_tau / sqrt(d), float64;
#  * y_t^(l) is the head-mean teacher mass of each non-current candidate's
#    subtree (tokens [u C^l, (u+1) C^l) clipped at t), renormalised over
#    those candidates: the support of pi_t^(l), the walk's importance (R4);
#  * only scored levels (|A| > k) contribute, where pi is defined;
#  * the shift penalty of level l averages over every complete level-l node
#    of every KV head (M_l of them): one pooler serves the layer.
# --------------------------------------------------------------------------

def teacher_attention(qG, t: int, K0, theta: float):
    """Dense attention probabilities [G, t+1] of the G query heads at t over
    the level-0 keys K0[0..t] (pre-RoPE), exact float64 RoPE."""
    qG = np.asarray(qG, dtype=np.float64)
    d = qG.shape[1]
    qr = rotate_exact(qG, t, theta)
    kr = rotate_exact(np.asarray(K0[: t + 1], dtype=np.float64), np.arange(t + 1), theta)
    s = (qr @ kr.T) / math.sqrt(d)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def subtree_mass(a, nodes, level: int, C: int):
    """Sum of a[..., tau] over the tokens under each node of ``level``:
    tau in [u C^level, (u+1) C^level), clipped at the end of a."""
    span = C ** level
    n_tok = a.shape[-1]
    out = np.zeros(a.shape[:-1] + (len(nodes),))
    for i, u in enumerate(nodes):
        lo, hi = int(u) * span, min((int(u) + 1) * span, n_tok)
        if lo < hi:
            out[..., i] = a[..., lo:hi].sum(axis=-1)
    return out


def distill_targets(qG, t: int, tr: WalkTrace, K0, C: int, theta: float):
    """The teacher distributions y_t^(l) of one query: {level: y} over the
    walk's scored levels, y[i] for the i-th non-current candidate of A^(l)."""
    a = teacher_attention(qG, t, K0, theta)
    out = {}
    for lvl, lt in tr.levels.items():
        if not lt.scored:
            continue
        m = subtree_mass(a, lt.A[:-1], lvl, C).mean(axis=0)
        out[lvl] = m / m.sum()
    return out


def distill_kl(qG, t: int, tr: WalkTrace, K0, C: int, theta: float):
    """Eq. 6 terms of one query: {level: KL(y || pi)} over the walk's scored
    levels, with 0 log 0 = 0."""
    out = {}
    for lvl, y in distill_targets(qG, t, tr, K0, C, theta).items():
        pi = np.asarray(tr.levels[lvl].importance, dtype=np.float64)
        nz = y > 0
        out[lvl] = float(np.sum(y[nz] * (np.log(y[nz]) - np.log(pi[nz]))))
    return out


def shift_penalty(children_by_level, P: Pooler):
    """Eq. 7 per level: ||mean_i sigma_i m_i||^2 / mean_i ||mu_i||^2 over the
    nodes i of that level.  children_by_level: {level: X [M_l, C, d]} -- the
    stored children of every complete node of the level (all KV heads)."""
    out = {}
    for lvl, X in children_by_level.items():
        mu, sigma, _, m = pool_parts(X, P)
        num = (sigma[:, None] * m).mean(axis=0)
        out[lvl] = float(num @ num / (mu * mu).sum(axis=1).mean())
    return out


# --------------------------------------------------------------------------
# Pooler backward (picx.dev "Pooler Distillation", Eq. 5 trained with Eq. 6
# and Eq. 7; "Training Stages", stage 1).  The vector-Jacobian product of
# Eq. 5 with respect to the pooler parameters, for a batch of nodes whose
# children are inputs (no gradient flows into the children: every level is
# pooled from stored, rounded rows).  Storage rounding of the node key is
# taken as the identity in the backward pass.
# --------------------------------------------------------------------------

def pool_backward(X, P: Pooler, dK, dm_extra=None):
    """Gradients of  L = sum_i dK_i . K_i + sum_i dm_extra_i . m_i  with
    respect to (w, tau, g, W1, b1, W2), K_i and m_i as in ``pool_parts``.
    X: [N, C, d] children; dK, dm_extra: [N, d].  Returns a dict of arrays
    shaped like the parameters (tau and g as floats)."""
    P = P.as64()
    X = np.asarray(X, dtype=np.float64)
    d = X.shape[2]
    # forward, keeping what the chain rule needs
    mu = X.mean(axis=1)
    dev = X - mu[:, None, :]
    sigma = np.sqrt((dev * dev).mean(axis=(1, 2)) + P.eps)
    rho = np.sqrt((mu * mu).mean(axis=1) + P.eps)
    u = (dev @ P.w) / sigma[:, None]                         # w.(x_c - mu)/sigma
    a = P.tau * u
    a = a - a.max(axis=1, keepdims=True)
    e = np.exp(a)
    alpha = e / e.sum(axis=1, keepdims=True)
    p = np.einsum("nc,ncd->nd", alpha, X)
    feat = np.concatenate([mu / rho[:, None], (p - mu) / sigma[:, None]], axis=1)
    z = feat @ P.W1.T + P.b1
    sg = 1.0 / (1.0 + np.exp(-z))
    hid = z * sg
    # backward: K = mu + g (p - mu) + sigma m,  m = W2 SiLU(z),  z = W1 feat + b1
    dK = np.asarray(dK, dtype=np.float64)
    dm = sigma[:, None] * dK
    if dm_extra is not None:
        dm = dm + np.asarray(dm_extra, dtype=np.float64)
    g_g = float(np.sum(dK * (p - mu)))
    g_W2 = dm.T @ hid                                         # [d, h]
    dz = (dm @ P.W2) * (sg * (1.0 + z * (1.0 - sg)))          # SiLU'(z)
    g_W1 = dz.T @ feat                                        # [h, 2d]
    g_b1 = dz.sum(axis=0)
    dfeat = dz @ P.W1                                         # [N, 2d]
    dp = P.g * dK + dfeat[:, d:] / sigma[:, None]             # mu/rho does not depend on
    dalpha = np.einsum("nd,ncd->nc", dp, X)                   # the parameters
    da = alpha * (dalpha - (alpha * dalpha).sum(axis=1, keepdims=True))
    g_tau = float(np.sum(da * u))
    g_w = P.tau * np.einsum("nc,ncd->d", da, dev / sigma[:, None, None])
    return {"w": g_w, "tau": g_tau, "g": g_g, "W1": g_W1, "b1": g_b1, "W2": g_W2}


def shift_penalty_dm(X, P: Pooler):
    """Gradient of the Eq. 7 penalty of one level with respect to each node's
    MLP output m_i (the only part of the penalty the parameters reach):
    with S = sum_i sigma_i m_i and U = sum_i ||mu_i||^2 over the level's M
    nodes, penalty = ||S||^2 / (M U), so d penalty / d m_i = 2 sigma_i S / (M U)."""
    mu, sigma, _, m = pool_parts(X, P)
    S = (sigma[:, None] * m).sum(axis=0)
    U = float((mu * mu).sum())
    M = X.shape[0]
    return 2.0 * sigma[:, None] * S[None, :] / (M * U)


def kl_key_grad(qG, t: int, tr: WalkTrace, K0, C: int, theta: float, cos=None, sin=None,
                dtype: str = "f32", exact: bool = False, magnitude: bool = False):
    """Gradient of one query's Eq. 6 terms, sum over scored levels of
    KL(y^(l) || pi^(l)), with respect to the stored key of every non-current
    candidate: {level: (nodes [n], dK [n, d])}.

    y does not depend on the tree (the teacher reads level-0 tokens only);
    pi = mean_h softmax_h(s_h) over the non-current candidates, so with
    r = y / pi and P_h = softmax_h(s_h),
        d KL / d s_h,e = -(P_h,e / G) (r_e - sum_f r_f P_h,f),
    and s_h,e = q~_h . k~_e / sqrt(d) gives d s / d K_e = R(c_e)^T q~_h / sqrt(d)
    in the split form (the operand roundings taken as the identity, the same
    float32 table entries), or R(p_q - p_e) q_h / sqrt(d) in exact mode.
    With magnitude, each term is replaced by its size without cancellation,
    (P_h,e / G)(|r_e| + |sum_f r_f P_h,f|) |R^T q~_h| / sqrt(d), which bounds
    how far a computation with relative error eps per input can move it."""
    ys = distill_targets(qG, t, tr, K0, C, theta)
    qG = np.asarray(qG, dtype=np.float64)
    G, d = qG.shape
    h = d // 2
    out = {}
    for lvl, y in ys.items():
        lt = tr.levels[lvl]
        others = lt.A[:-1]
        n = len(others)
        s = np.asarray(lt.logits, dtype=np.float64)                 # [G, n]
        P = np.exp(s - s.max(axis=1, keepdims=True))
        P = P / P.sum(axis=1, keepdims=True)
        r = y / P.mean(axis=0)
        S = (P * r[None, :]).sum(axis=1, keepdims=True)
        coef = -(P / G) * (r[None, :] - S)
        if magnitude:
            coef = (P / G) * (np.abs(r[None, :]) + np.abs(S))
        p_q = len(lt.A) - 1
        pos_e = np.arange(n)
        if exact:
            qrot = rotate_exact(qG[:, None, :], (p_q - pos_e)[None, :], theta)   # [G, n, d]
        else:
            r_q, c_q = divmod(p_q, C)
            r_e, c_e = pos_e // C, pos_e % C
            qt = np.empty((G, n, d))
            for rr in np.unique(r_e):
                idx = np.nonzero(r_e == rr)[0]
                phi = C * (r_q - int(rr)) + c_q
                qt[:, idx] = rnd(rotate_f32(qG, cos[phi], sin[phi]).astype(np.float64),
                                 dtype)[:, None, :]
            cc = cos[c_e].astype(np.float64)[None]                   # [1, n, d/2]
            ss = sin[c_e].astype(np.float64)[None]
            x, yv = qt[..., :h], qt[..., h:]
            qrot = np.concatenate([x * cc + yv * ss, -x * ss + yv * cc], axis=-1)  # R(c)^T q~
        if magnitude:
            qrot = np.abs(qrot)
        out[lvl] = (others, np.einsum("gn,gnd->nd", coef, qrot) / math.sqrt(d))
    return out
