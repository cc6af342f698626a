"""Pins of the CPU oracle against what the pages and mathematics fix.

Every check here is independent of the oracle's own formulas: closed forms,
invariants, special cases that reduce to a library routine (torch SDPA, scipy
softmax, torch bf16 conversion, torch SiLU), brute force on tiny inputs, and
the structural numbers the pages print (tests/golden/pages_structural.json).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import recsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_structural.json")


def _pooler(d, h, seed, **over):
    r = np.random.default_rng(seed)
    P = dict(w=r.standard_normal(d) / math.sqrt(d), tau=1.0, g=0.5,
             W1=r.standard_normal((h, 2 * d)) / math.sqrt(d),
             b1=r.standard_normal(h) / math.sqrt(d),
             W2=r.standard_normal((d, h)) / math.sqrt(d), eps=1e-6)
    P.update(over)
    return O.Pooler(**P)


def _tree(L, d, C, k, seed, dtype="f32", n_levels=None, h=None):
    r = np.random.default_rng(seed)
    K0 = r.standard_normal((L, d))
    V0 = r.standard_normal((L, d))
    D = n_levels or O.n_levels_for(L - 1, C, k)
    P = _pooler(d, h or d, seed + 1)
    K, V = O.build_tree(K0, V0, C, D, P, dtype)
    return K, V, P


def _complex_rope(v, pos, theta):
    """Textbook RoPE as complex multiplication: pair (j, j+d/2) is the complex
    number v_j + i v_{j+d/2}, multiplied by exp(i pos theta^(-2j/d))."""
    d = v.shape[-1]
    h = d // 2
    z = v[..., :h] + 1j * v[..., h:]
    w = float(theta) ** (-2.0 * np.arange(h) / d)
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * w)
    return np.concatenate([z.real, z.imag], axis=-1)


# --------------------------------------------------------------------------
# storage rounding and RoPE tables
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch():
    r = np.random.default_rng(0)
    x = (r.standard_normal(200000) * np.exp(r.uniform(-80, 80, 200000))).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                                     2.0 ** -130, -(2.0 ** -131)], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_rope_table_group_property_and_base():
    d, n, theta = 64, 4096, 1e6
    cos, sin = O.rope_table(d, n, theta)
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)
    # pair 0 turns by exactly one radian per position
    assert np.allclose(cos[:, 0], np.cos(np.arange(n)), atol=6e-8)
    # R(a) R(b) = R(a + b) up to float32 rounding of the table
    a, b = 1234, 2000
    ca, sa, cb, sb = (cos[a].astype(np.float64), sin[a].astype(np.float64),
                      cos[b].astype(np.float64), sin[b].astype(np.float64))
    assert np.allclose(ca * cb - sa * sb, cos[a + b], atol=3e-7)
    assert np.allclose(sa * cb + ca * sb, sin[a + b], atol=3e-7)
    # lowest frequency is theta^(-(d-2)/d)
    w_last = theta ** (-(d - 2) / d)
    assert np.allclose(sin[1:50, -1], np.sin(np.arange(1, 50) * w_last), atol=1e-9)


def test_rotate_f32_error_bound_vs_complex_rope():
    r = np.random.default_rng(1)
    d, theta = 128, 1e6
    cos, sin = O.rope_table(d, 4096, theta)
    v = r.standard_normal((4096, d)).astype(np.float32)
    pos = np.arange(4096)
    got = O.rotate_f32(v, cos[pos], sin[pos]).astype(np.float64)
    ref = _complex_rope(v.astype(np.float64), pos, theta)
    h = d // 2
    bound = (np.abs(v[:, :h]) + np.abs(v[:, h:])).astype(np.float64) * 2.0 ** -22
    err = np.abs(got - ref)
    assert np.all(err[:, :h] <= bound) and np.all(err[:, h:] <= bound)
    # exact-mode rotation is the complex rotation
    assert np.allclose(O.rotate_exact(v, pos, theta), ref, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# Eq. 1 values and Eq. 5 pooler
# --------------------------------------------------------------------------

def test_node_value_is_subtree_mean():
    """P1: a node's value is the mean of every token in its subtree
    (picx.dev Eq. 1; kongchang article: node value = mean of all token values
    in the subtree)."""
    C, L, d = 4, 4 ** 4, 8
    K, V, _ = _tree(L, d, C, 4, 3, "f32", n_levels=5)
    V0 = V[0]
    for lvl in range(1, 5):
        span = C ** lvl
        ref = V0.reshape(-1, span, d).mean(axis=1)
        assert np.allclose(V[lvl], ref, rtol=0, atol=lvl * 2.0 ** -22)
    # bf16 storage: each level adds at most half a bf16 ulp of a value no
    # larger than the largest token of the subtree
    K, V, _ = _tree(L, d, C, 4, 3, "bf16", n_levels=5)
    for lvl in range(1, 5):
        sub = V[0].reshape(-1, C ** lvl, d)
        ref = sub.mean(axis=1)
        bound = lvl * 2.0 ** -8 * np.abs(sub).max(axis=1)
        assert np.all(np.abs(V[lvl] - ref) <= bound)


def test_pooler_permutation_invariant():
    r = np.random.default_rng(5)
    P = _pooler(16, 16, 6)
    X = r.standard_normal((7, 16, 16))
    perm = r.permutation(16)
    assert np.allclose(O.pool_keys(X, P), O.pool_keys(X[:, perm], P), atol=1e-12)


def test_pooler_shift_and_scale_equivariance_without_mlp():
    r = np.random.default_rng(7)
    d = 16
    P = _pooler(d, d, 8, W2=np.zeros((d, d)), eps=0.0)
    X = r.standard_normal((5, 16, d))
    b = r.standard_normal(d)
    assert np.allclose(O.pool_keys(X + b, P), O.pool_keys(X, P) + b, atol=1e-12)
    assert np.allclose(O.pool_keys(3.5 * X, P), 3.5 * O.pool_keys(X, P), atol=1e-12)


def test_pooler_reduces_to_mean_and_argmax():
    r = np.random.default_rng(9)
    d = 8
    X = r.standard_normal((6, 16, d))
    # g = 0 and W2 = 0: the key is the children mean
    P = _pooler(d, d, 10, g=0.0, W2=np.zeros((d, d)))
    assert np.allclose(O.pool_keys(X, P), X.mean(axis=1), atol=1e-12)
    # tau = 0: alpha uniform, p = mu, so with W2 = 0 the key is the mean for any g
    P = _pooler(d, d, 10, tau=0.0, g=0.7, W2=np.zeros((d, d)))
    assert np.allclose(O.pool_keys(X, P), X.mean(axis=1), atol=1e-12)
    # very large tau: p is the child with the largest w.x (textbook argmax)
    P = _pooler(d, d, 10, tau=1e6, g=1.0, W2=np.zeros((d, d)))
    best = np.argmax(X @ P.w, axis=1)
    assert np.allclose(O.pool_keys(X, P), X[np.arange(6), best], atol=1e-9)


def test_pooler_attention_weights_are_softmax_over_children():
    """p = sum softmax_c(tau w.(x_c - mu)/sigma) x_c with sigma the population
    standard deviation of the child entries around the per-dim mean (scipy
    softmax, numpy var)."""
    r = np.random.default_rng(11)
    d, tau = 8, 1.7
    X = r.standard_normal((4, 16, d))
    w = np.zeros(d)
    w[0] = 1.0
    P = _pooler(d, d, 12, w=w, tau=tau, g=1.0, W2=np.zeros((d, d)), eps=0.0)
    sigma = np.sqrt(np.var(X, axis=1).mean(axis=1))
    z = X[:, :, 0] - X[:, :, 0].mean(axis=1, keepdims=True)
    alpha = scipy.special.softmax(tau * z / sigma[:, None], axis=1)
    ref = np.einsum("nc,ncd->nd", alpha, X)
    assert np.allclose(O.pool_keys(X, P), ref, atol=1e-12)


def test_pooler_mlp_input_order_and_output_orientation():
    r = np.random.default_rng(13)
    d, h = 8, 6
    X = r.standard_normal((3, 16, d))
    X[:, :, 0] -= X[:, :, 0].mean(axis=1, keepdims=True)     # mu_0 = 0
    # W1 reads only feature 0 of the concatenation; that is mu_0/rho = 0, so
    # with b1 = 0 the hidden layer is SiLU(0) = 0 and m = 0
    W1 = np.zeros((h, 2 * d))
    W1[:, 0] = 1.0
    P = _pooler(d, h, 14, W1=W1, b1=np.zeros(h))
    P0 = _pooler(d, h, 14, W2=np.zeros((d, h)))
    assert np.allclose(O.pool_keys(X, P), O.pool_keys(X, P0), atol=1e-12)
    # W2 with a single entry (row 2, column 4) moves only output dim 2
    W2 = np.zeros((d, h))
    W2[2, 4] = 1.0
    P = _pooler(d, h, 14, W2=W2)
    diff = O.pool_keys(X, P) - O.pool_keys(X, P0)
    assert np.all(np.abs(np.delete(diff, 2, axis=1)) < 1e-12)
    assert np.all(np.abs(diff[:, 2]) > 1e-6)


def test_pooler_mlp_term_is_sigma_times_silu():
    """With tau = 0 (p = mu), g arbitrary, children whose mean is a*1, W1
    reading mu_0/rho (= a/sqrt(a^2+eps)) and W2 with one entry, the key's dim 0
    is mu_0 + sigma * SiLU(a/sqrt(a^2 + eps) + beta) (torch SiLU)."""
    r = np.random.default_rng(15)
    d, h, eps = 8, 4, 1e-6
    for a, beta in [(0.3, 0.0), (-1.2, 0.5), (2.0, -3.0), (0.05, 1.0)]:
        dev = r.standard_normal((1, 16, d))
        dev -= dev.mean(axis=1, keepdims=True)
        X = a + dev
        W1 = np.zeros((h, 2 * d))
        W1[1, 0] = 1.0
        b1 = np.zeros(h)
        b1[1] = beta
        W2 = np.zeros((d, h))
        W2[0, 1] = 1.0
        P = _pooler(d, h, 16, tau=0.0, g=0.3, W1=W1, b1=b1, W2=W2, eps=eps)
        sigma = math.sqrt(np.var(X[0], axis=0).mean() + eps)
        u = a / math.sqrt(a * a + eps) + beta
        silu = torch.nn.functional.silu(torch.tensor(u, dtype=torch.float64)).item()
        got = O.pool_keys(X, P)[0]
        assert got[0] == pytest.approx(a + sigma * silu, abs=1e-12)
        assert np.allclose(got[1:], a, atol=1e-12)


def test_pooler_deviation_scaling_scales_mlp_term():
    """Scaling the children's deviations about a fixed mean by lam leaves
    mu/rho and (p - mu)/sigma unchanged (eps = 0), so K - mu - g(p - mu) =
    sigma*m scales by lam, as does p - mu."""
    r = np.random.default_rng(17)
    d = 8
    P = _pooler(d, d, 18, eps=0.0)
    Pg0 = _pooler(d, d, 18, eps=0.0, g=0.0)
    Pm0 = _pooler(d, d, 18, eps=0.0, g=0.0, W2=np.zeros((d, d)))
    mu = r.standard_normal((3, 1, d))
    dev = r.standard_normal((3, 16, d))
    dev -= dev.mean(axis=1, keepdims=True)
    lam = 2.5
    t1 = O.pool_keys(mu + dev, Pg0) - O.pool_keys(mu + dev, Pm0)        # sigma*m
    t2 = O.pool_keys(mu + lam * dev, Pg0) - O.pool_keys(mu + lam * dev, Pm0)
    assert np.allclose(t2, lam * t1, atol=1e-11)
    g1 = O.pool_keys(mu + dev, P) - O.pool_keys(mu + dev, Pg0)           # g(p - mu)
    g2 = O.pool_keys(mu + lam * dev, P) - O.pool_keys(mu + lam * dev, Pg0)
    assert np.allclose(g2, lam * g1, atol=1e-11)


# --------------------------------------------------------------------------
# Eq. 3 walk and Eq. 4 softmax
# --------------------------------------------------------------------------

TINY_CONFIGS = [(C, k, d) for C in (2, 3, 4, 16) for k in (1, 2, 3, 16) for d in (4,)]


def _positions_ok(tr, C, k):
    for lt in tr.levels.values():
        assert len(lt.A) <= C * k
    assert len(tr.A0) <= C * k


def _check_structure(tr, t, C, k):
    # P2: current node always selected, |S| = min(k, |A|), S subset of A
    for lvl, lt in tr.levels.items():
        cur = t // C ** lvl
        assert cur in set(lt.S.tolist())
        assert len(lt.S) == min(k, len(lt.A))
        assert set(lt.S.tolist()) <= set(lt.A.tolist())
        assert np.all(np.diff(lt.S) > 0)
    # P3: every list position (and so every distance to the query) < C*k
    _positions_ok(tr, C, k)
    # P6: the subtrees of E partition [0..t]
    cover = np.zeros(t + 1, dtype=np.int64)
    for lvl, node in tr.entries:
        span = C ** lvl
        lo, hi = node * span, (node + 1) * span
        assert hi <= t + 1 or lvl == 0
        cover[lo:min(hi, t + 1)] += 1
    assert np.all(cover == 1)
    # Eq. 3 third line, re-derived from the selections: A^(l-1) = children of S^(l)
    lvls = sorted(tr.levels)
    for lvl in lvls:
        below = tr.levels[lvl - 1].A if lvl - 1 in tr.levels else tr.A0
        want = [c for i in tr.levels[lvl].S.tolist()
                for c in range(C * i, min(C * i + C - 1, t // C ** (lvl - 1)) + 1)]
        assert below.tolist() == want


@pytest.mark.parametrize("C,k,d", TINY_CONFIGS)
def test_walk_structure_every_position(C, k, d):
    L = 300 if C > 2 else 200
    K, V, _ = _tree(L, d, C, k, 100 + C * 10 + k, "f32")
    cos, sin = O.rope_table(d, C * k, 1e6)
    r = np.random.default_rng(C * 100 + k)
    for t in range(L):
        q = r.standard_normal((2, d))
        D = O.n_levels_for(t, C, k)
        Kt = [K[0][: t + 1]] + [K[lvl][: (t + 1) // C ** lvl] for lvl in range(1, D)]
        tr = O.walk(q, t, Kt, C, k, cos, sin, "f32")
        _check_structure(tr, t, C, k)


def _dominance_ok(I, nodes, X):
    Xs = set(X)
    for x in X:
        for y in range(len(I)):
            if y in Xs:
                continue
            if not (I[x] > I[y] or (I[x] == I[y] and nodes[x] < nodes[y])):
                return False
    return True


@pytest.mark.parametrize("C,k", [(2, 2), (2, 3), (3, 2), (3, 3), (4, 2), (4, 3)])
def test_topk_brute_force(C, k):
    """P4: each scored level keeps exactly the unique subset of size k-1 that
    dominates every left-out candidate (found by enumerating all subsets)."""
    d = 4
    L = 300
    K, V, _ = _tree(L, d, C, k, 200 + C + k, "f32")
    cos, sin = O.rope_table(d, C * k, 1e6)
    r = np.random.default_rng(C * 7 + k)
    checked = 0
    for t in range(0, L, 3):
        q = r.standard_normal((3, d))
        D = O.n_levels_for(t, C, k)
        Kt = [K[0][: t + 1]] + [K[lvl][: (t + 1) // C ** lvl] for lvl in range(1, D)]
        tr = O.walk(q, t, Kt, C, k, cos, sin, "f32")
        for lvl, lt in tr.levels.items():
            if not lt.scored:
                continue
            others = lt.A[:-1]
            m = min(k - 1, len(others))
            valid = [X for X in itertools.combinations(range(len(others)), m)
                     if _dominance_ok(lt.importance, others, X)]
            assert len(valid) == 1
            got = sorted(set(lt.S.tolist()) - {int(lt.A[-1])})
            assert got == sorted(int(others[i]) for i in valid[0])
            checked += 1
    assert checked > 20


def test_topk_ties_pick_lowest_indices_and_plain_mean():
    """P9: zero level-0 keys with b1 = 0 make every node key zero, so all
    importances tie: the walk keeps the current node plus the k-1 lowest
    indices, and the output is the plain mean of the entry values."""
    C, k, d, L = 4, 3, 8, 256
    r = np.random.default_rng(19)
    K0 = np.zeros((L, d))
    V0 = r.standard_normal((L, d))
    P = _pooler(d, d, 20, b1=np.zeros(d))
    D = O.n_levels_for(L - 1, C, k)
    K, V = O.build_tree(K0, V0, C, D, P, "f32")
    cos, sin = O.rope_table(d, C * k, 1e6)
    t = L - 1
    tr = O.walk(r.standard_normal((2, d)), t, K, C, k, cos, sin, "f32")
    for lvl, lt in tr.levels.items():
        if lt.scored:
            assert lt.S.tolist() == lt.A[: k - 1].tolist() + [int(lt.A[-1])]
    o = O.attend(tr, V)
    rows = np.stack([V[lvl][node] for lvl, node in tr.entries])
    assert np.allclose(o, rows.mean(axis=0)[None, :], atol=1e-12)


def test_constant_values_give_constant_output():
    """P9: if every token value is the same vector, so is every node value
    and the output, whatever the selection."""
    C, k, d, L = 4, 3, 8, 300
    r = np.random.default_rng(21)
    K0 = r.standard_normal((L, d))
    V0 = np.tile(r.standard_normal(d), (L, 1))
    D = O.n_levels_for(L - 1, C, k)
    K, V = O.build_tree(K0, V0, C, D, _pooler(d, d, 22), "f32")
    cos, sin = O.rope_table(d, C * k, 1e6)
    o, _ = O.decode_reference(r.standard_normal((3, d)), L - 1, K, V, C, k, cos, sin, "f32")
    assert np.allclose(o, V0[0][None, :], atol=1e-12)


@pytest.mark.parametrize("exact", [True, False])
def test_short_context_equals_dense_rope_attention(exact):
    """P5: for t < C*k every level has at most k candidates, so the output is
    dense causal attention with RoPE at absolute positions (torch SDPA in
    float64, RoPE by complex multiplication)."""
    C, k, d, theta = 4, 8, 16, 1e4
    L = C * k
    r = np.random.default_rng(23)
    K0 = r.standard_normal((L, d))
    V0 = r.standard_normal((L, d))
    D = O.n_levels_for(L - 1, C, k)
    K, V = O.build_tree(K0, V0, C, D, _pooler(d, d, 24), "f32")
    cos, sin = O.rope_table(d, C * k, theta)
    for t in range(0, L, 5):
        q = r.standard_normal((4, d))
        Kt = [K[0][: t + 1]] + [K[lvl][: (t + 1) // C ** lvl] for lvl in range(1, D)]
        o, tr = O.decode_reference(q, t, Kt, V, C, k, cos, sin, "f32", exact=exact,
                                   theta=theta)
        qr = _complex_rope(q, np.full(4, t), theta)
        kr = _complex_rope(K[0][: t + 1], np.arange(t + 1), theta)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qr)[None, :, None, :],
            torch.from_numpy(np.broadcast_to(kr, (4, t + 1, d)).copy())[None],
            torch.from_numpy(np.broadcast_to(V[0][: t + 1], (4, t + 1, d)).copy())[None],
        )[0, :, 0].numpy()
        tol = 1e-12 if exact else 2e-6
        assert np.allclose(o, ref, atol=tol, rtol=0), (t, np.abs(o - ref).max())


def test_split_logits_equal_candidate_local_rope():
    """The split form (query turned by C*(r_q - r_e) + c_q, key by c_e) equals
    RoPE at the candidate-local positions: exact mode vs float32 split."""
    C, k, d, L = 16, 16, 64, 4096
    K, V, _ = _tree(L, d, C, k, 25, "f32")
    cos, sin = O.rope_table(d, C * k, 1e6)
    r = np.random.default_rng(26)
    for t in (4095, 3000, 1234):
        q = r.standard_normal((4, d))
        Kt = [K[0][: t + 1]] + [K[lvl][: (t + 1) // C ** lvl] for lvl in range(1, len(K))]
        a = O.walk(q, t, Kt, C, k, cos, sin, "f32")
        b = O.walk(q, t, Kt, C, k, exact=True)
        for lvl in a.levels:
            if a.levels[lvl].scored:
                assert np.allclose(a.levels[lvl].logits, b.levels[lvl].logits, atol=2e-5)
        if [lt.S.tolist() for lt in a.levels.values()] == [lt.S.tolist() for lt in b.levels.values()]:
            assert np.allclose(a.entry_logits, b.entry_logits, atol=2e-5)


def test_k1_selects_canonical_coarsest_cover():
    """P11: with k = 1 the walk keeps only the current node, so E is the
    greedy cover of [0..t] by the largest aligned blocks that end before t,
    plus the exact tokens from the last block start to t."""
    C, d = 3, 4
    K, V, _ = _tree(250, d, C, 1, 27, "f32", n_levels=O.n_levels_for(249, C, 1))
    cos, sin = O.rope_table(d, C, 1e6)
    for t in range(250):
        D = O.n_levels_for(t, C, 1)
        Kt = [K[0][: t + 1]] + [K[lvl][: (t + 1) // C ** lvl] for lvl in range(1, D)]
        tr = O.walk(np.ones((1, d)), t, Kt, C, 1, cos, sin, "f32")
        want, pos = [], 0
        while pos <= t:
            lvl = D - 1
            while lvl > 0 and not (pos % C ** lvl == 0 and pos + C ** lvl - 1 < t):
                lvl -= 1
            want.append((lvl, pos // C ** lvl))
            pos += C ** lvl
        assert sorted(tr.entries) == sorted(want)


def test_extra_level_changes_nothing():
    """P12: building and walking one level more than needed gives identical
    selections, entries and logits."""
    C, k, d, L = 4, 3, 8, 300
    r = np.random.default_rng(29)
    K0, V0 = r.standard_normal((L, d)), r.standard_normal((L, d))
    P = _pooler(d, d, 30)
    D = O.n_levels_for(L - 1, C, k)
    Ka, Va = O.build_tree(K0, V0, C, D, P, "f32")
    Kb, Vb = O.build_tree(K0, V0, C, D + 2, P, "f32")
    cos, sin = O.rope_table(d, C * k, 1e6)
    q = r.standard_normal((2, d))
    oa, ta = O.decode_reference(q, L - 1, Ka, Va, C, k, cos, sin, "f32")
    ob, tb = O.decode_reference(q, L - 1, Kb, Vb, C, k, cos, sin, "f32")
    assert ta.entries == tb.entries
    assert np.array_equal(ta.entry_logits, tb.entry_logits)
    assert np.array_equal(oa, ob)


def test_single_head_importance_ranks_by_logit():
    """P13: with one query head the softmax is monotone, so the selection is
    the current node plus the k-1 largest logits."""
    C, k, d, L = 4, 3, 8, 300
    K, V, _ = _tree(L, d, C, k, 31, "f32")
    cos, sin = O.rope_table(d, C * k, 1e6)
    r = np.random.default_rng(32)
    for t in range(100, L, 7):
        tr = O.walk(r.standard_normal((1, d)), t, K, C, k, cos, sin, "f32")
        for lt in tr.levels.values():
            if lt.scored:
                s = lt.logits[0]
                order = np.lexsort((lt.A[:-1], -s))[: k - 1]
                assert sorted(lt.A[:-1][order].tolist() + [int(lt.A[-1])]) == lt.S.tolist()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_equals_rebuild(dtype):
    """P-append: appending tokens one by one (completing nodes as their last
    token arrives) equals a full rebuild, bit for bit."""
    C, k, d = 4, 3, 8
    r = np.random.default_rng(33)
    K0, V0 = r.standard_normal((200, d)), r.standard_normal((200, d))
    P = _pooler(d, d, 34)
    D = 4
    K, V = O.build_tree(K0[:37], V0[:37], C, D, P, dtype)
    for t in range(37, 200):
        K, V = O.append_token(K, V, K0[t], V0[t], C, P, dtype)
    Kr, Vr = O.build_tree(K0, V0, C, D, P, dtype)
    for lvl in range(D):
        assert np.array_equal(K[lvl], Kr[lvl]) and np.array_equal(V[lvl], Vr[lvl])


def test_published_token_budget_and_overhead():
    """P7/P8: at L = 10^6 with C = 16, k = 256 the entry count is data-free;
    it reproduces the pages' 1.16% token budget.  Levels above 0 add
    sum_l 16^-l -> 1/15 of the cache, under the pages' 7%."""
    gold = json.load(open(GOLDEN))
    C, k = gold["branching_C"]["value"], gold["budget_k"]["value"]
    L = gold["token_budget_1M_percent"]["context"]
    d = 4
    t = L - 1
    D = O.n_levels_for(t, C, k)
    r = np.random.default_rng(35)
    K0 = r.standard_normal((L, d))
    K, V = O.build_tree(K0, K0, C, D, _pooler(d, d, 36), "f32")
    cos, sin = O.rope_table(d, C * k, 1e6)
    tr = O.walk(r.standard_normal((1, d)), t, K, C, k, cos, sin, "f32")
    sizes = [len(tr.levels[lvl].A) for lvl in sorted(tr.levels, reverse=True)] + [len(tr.A0)]
    assert sizes == [245, 3907, 4084, 4096]
    n_e = len(tr.entries)
    assert n_e == 11575
    assert round(100.0 * n_e / L, 2) == gold["token_budget_1M_percent"]["value"]
    assert max(sizes) <= gold["position_bound"]["value"] == C * k
    for L2 in (131072, 524288, 1048576, 2097152):
        sizes = O.level_sizes(L2, C, O.n_levels_for(L2 - 1, C, k) + 1)
        frac = sum(sizes[1:]) / L2
        assert frac < gold["tree_overhead_bound_percent"]["value"] / 100
        assert abs(frac - 1 / 15) < 1e-3


# --------------------------------------------------------------------------
# pooler distillation losses (Eq. 6, Eq. 7)
# --------------------------------------------------------------------------

def test_teacher_attention_is_sdpa_with_textbook_rope():
    """The teacher's probabilities are torch SDPA (causal row t) on queries
    and keys rotated as complex numbers, read out with one-hot values."""
    r = np.random.default_rng(71)
    d, t, theta = 16, 40, 1e4
    K0 = r.standard_normal((t + 1, d))
    q = r.standard_normal((3, d))
    a = O.teacher_attention(q, t, K0, theta)
    qr = torch.tensor(_complex_rope(q, np.full(3, t), theta))[None, :, None, :]    # [1, G, 1, d]
    kr = torch.tensor(_complex_rope(K0, np.arange(t + 1), theta))[None, None].expand(1, 3, t + 1, d)
    eye = torch.eye(t + 1, dtype=torch.float64)[None, None].expand(1, 3, t + 1, t + 1)
    ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, eye)[0, :, 0].numpy()
    assert np.allclose(a, ref, rtol=0, atol=1e-12)
    assert np.allclose(a.sum(axis=1), 1.0)
    # a single token takes all the mass; equal keys give uniform attention
    assert np.allclose(O.teacher_attention(q, 0, K0, theta), 1.0)
    flat = O.teacher_attention(q, t, np.zeros((t + 1, d)), theta)
    assert np.allclose(flat, 1.0 / (t + 1))


def test_subtree_masses_partition_the_tokens():
    r = np.random.default_rng(72)
    a = r.random((2, 300))
    a /= a.sum(axis=1, keepdims=True)
    for lvl, C in ((1, 4), (2, 4), (1, 16), (2, 3)):
        n_nodes = -(-300 // C ** lvl)
        m = O.subtree_mass(a, np.arange(n_nodes), lvl, C)
        assert np.allclose(m.sum(axis=1), 1.0)
        assert np.allclose(m[:, 0], a[:, :C ** lvl].sum(axis=1))


def test_distill_kl_zero_for_zero_query_and_matches_relative_entropy():
    """q = 0: the teacher is uniform over tokens, so the non-current
    candidates (complete subtrees of equal size) get uniform y, and every
    logit is 0, so pi is uniform too: KL = 0 at every scored level.  For
    random queries each term is scipy's relative entropy of (y, pi) and >= 0."""
    C, k, d, L = 4, 3, 8, 300
    K, V, P = _tree(L, d, C, k, 73, "f32")
    cos, sin = O.rope_table(d, C * k, 1e4)
    t = L - 1
    q0 = np.zeros((2, d))
    tr0 = O.walk(q0, t, K, C, k, cos, sin, "f32", theta=1e4)
    kl0 = O.distill_kl(q0, t, tr0, K[0], C, 1e4)
    assert kl0 and all(abs(v) < 1e-14 for v in kl0.values())
    r = np.random.default_rng(74)
    for _ in range(4):
        q = r.standard_normal((2, d))
        tr = O.walk(q, t, K, C, k, cos, sin, "f32", theta=1e4)
        kl = O.distill_kl(q, t, tr, K[0], C, 1e4)
        a = O.teacher_attention(q, t, K[0], 1e4)
        for lvl, v in kl.items():
            lt = tr.levels[lvl]
            m = O.subtree_mass(a, lt.A[:-1], lvl, C).mean(axis=0)
            assert v >= 0
            assert abs(v - scipy.stats.entropy(m / m.sum(), lt.importance)) < 1e-12


def test_distill_targets_average_heads_then_renormalise():
    """R15 by hand: head 0 with q = 0 spreads the teacher mass uniformly
    over the t+1 tokens; head 1 puts all of it on one token tau* (its query
    is the RoPE-rotated key of an outsized token).  Per candidate u of a
    scored level (n_u tokens in its subtree, the current node dropped) the
    head-mean mass is m_u = (n_u/(t+1) + [tau* under u]) / 2, and y is m
    renormalised over the candidates.  Normalising each head first and then
    averaging, or keeping the current node, would give other values."""
    C, k, d, L, theta = 4, 3, 8, 300, 1e4
    r = np.random.default_rng(76)
    K0 = r.standard_normal((L, d))
    t = L - 1
    K, V, P = _tree(L, d, C, k, 77, "f32")
    cos, sin = O.rope_table(d, C * k, theta)
    # the candidate lists come from some walk; the teacher from the two heads
    tr = O.walk(r.standard_normal((2, d)), t, K, C, k, cos, sin, "f32", theta=theta)
    lowest = min(l for l, lt in tr.levels.items() if lt.scored)
    lt0 = tr.levels[lowest]
    u_star = int(lt0.A[len(lt0.A) // 2])            # a non-current candidate
    tau_star = u_star * C ** lowest + 1
    K0[tau_star] *= 30.0
    q1 = 40.0 * O.rotate_exact(K0[tau_star], tau_star - t, theta)
    qG = np.stack([np.zeros(d), q1])
    a = O.teacher_attention(qG, t, K0, theta)
    assert np.allclose(a[0], 1.0 / (t + 1)) and a[1, tau_star] == 1.0
    y = O.distill_targets(qG, t, tr, K0, C, theta)
    discriminating = 0
    for lvl, lt in tr.levels.items():
        if not lt.scored:
            assert lvl not in y
            continue
        span = C ** lvl
        nodes = lt.A[:-1]
        n_u = np.array([min((u + 1) * span, t + 1) - u * span for u in nodes], dtype=np.float64)
        hit = np.array([u * span <= tau_star < (u + 1) * span for u in nodes], dtype=np.float64)
        m = 0.5 * (n_u / (t + 1) + hit)
        assert np.allclose(y[lvl], m / m.sum(), rtol=0, atol=1e-15), lvl
        if hit.any():
            discriminating += 1
            per_head_first = 0.5 * (n_u / n_u.sum() + hit)
            assert np.abs(per_head_first - y[lvl]).max() > 1e-3
    assert discriminating >= 1


def test_pooler_sigma_is_one_scalar_over_children_and_dims():
    """R8 reads sigma as one population standard deviation over all C x d
    child entries.  Without the MLP (W2 = 0) and with g = 1 the key is the
    attention-pooled child p, whose softmax logits tau w.(x_c - mu)/sigma
    depend on sigma.  Rotating every child's deviation from mu by one
    orthogonal matrix Q (and w with it) leaves a scalar over all entries
    unchanged, so the key is Q-rotated exactly; a per-dimension or a
    per-child deviation would not be invariant.  Scaling one dimension's
    deviations by 3 changes the scalar sigma and hence the pooling weights."""
    r = np.random.default_rng(78)
    d, n = 8, 5
    X = r.standard_normal((n, 16, d))
    w = r.standard_normal(d)
    Q, _ = np.linalg.qr(r.standard_normal((d, d)))
    P = _pooler(d, d, 79, w=w, tau=2.0, g=1.0, W2=np.zeros((d, d)), eps=0.0)
    Pq = _pooler(d, d, 79, w=Q @ w, tau=2.0, g=1.0, W2=np.zeros((d, d)), eps=0.0)
    mu = X.mean(axis=1, keepdims=True)
    Xq = mu + (X - mu) @ Q.T
    k1 = O.pool_keys(X, P)
    k2 = O.pool_keys(Xq, Pq)
    assert np.allclose(k2 - mu[:, 0], (k1 - mu[:, 0]) @ Q.T, atol=1e-12)
    # with a one-hot w, only dimension 0 enters the logits: stretching
    # dimension 5's deviations changes sigma (a scalar over all entries) and
    # therefore the weights, which a per-dimension sigma would not do
    e0 = np.zeros(d)
    e0[0] = 1.0
    P0 = _pooler(d, d, 79, w=e0, tau=2.0, g=1.0, W2=np.zeros((d, d)), eps=0.0)
    Xs = X.copy()
    Xs[:, :, 5] = mu[:, :, 5] + 3.0 * (X[:, :, 5] - mu[:, :, 5])
    ks, k0 = O.pool_keys(Xs, P0), O.pool_keys(X, P0)
    assert np.abs(ks[:, 0] - k0[:, 0]).max() > 1e-3


def test_shift_penalty_invariants():
    """Eq. 7: zero without the MLP term (W2 = 0); unchanged by scaling every
    child key by c > 0 (sigma and mu scale by c, m does not) up to eps, and
    by the order of the nodes; one node gives ||sigma m||^2 / ||mu||^2."""
    r = np.random.default_rng(75)
    d, h, C = 8, 8, 4
    X = r.standard_normal((30, C, d)) + 0.3
    P = _pooler(d, h, 76)
    base = O.shift_penalty({1: X}, P)[1]
    assert base > 0
    assert O.shift_penalty({1: X}, _pooler(d, h, 76, W2=np.zeros((d, h))))[1] == 0.0
    P0 = _pooler(d, h, 76, eps=0.0)
    base0 = O.shift_penalty({1: X}, P0)[1]
    for c in (0.5, 7.0):
        # exact without eps; with eps = 1e-6 inside the roots, within 1e-4
        assert abs(O.shift_penalty({1: c * X}, P0)[1] - base0) < 1e-12 * base0
        assert abs(O.shift_penalty({1: c * X}, P)[1] - base) < 1e-4 * base
    perm = r.permutation(30)
    assert abs(O.shift_penalty({1: X[perm]}, P)[1] - base) < 1e-12 * base
    mu, sigma, _, m = O.pool_parts(X[:1], P)
    one = O.shift_penalty({1: X[:1]}, P)[1]
    assert abs(one - np.sum((sigma[0] * m[0]) ** 2) / np.sum(mu[0] ** 2)) < 1e-12 * one


def _fd_grads(loss, P, step=1e-6, picks=None):
    """Central differences of loss(P) for every parameter entry (or the
    entries listed in picks[name])."""
    out = {}
    for name in ("w", "W1", "b1", "W2"):
        arr = getattr(P, name)
        g = np.zeros_like(arr)
        idx = picks[name] if picks and name in picks else list(np.ndindex(arr.shape))
        for ix in idx:
            old = arr[ix]
            arr[ix] = old + step
            fp = loss(P)
            arr[ix] = old - step
            fm = loss(P)
            arr[ix] = old
            g[ix] = (fp - fm) / (2 * step)
        out[name] = (g, idx)
    for name in ("tau", "g"):
        old = getattr(P, name)
        setattr(P, name, old + step)
        fp = loss(P)
        setattr(P, name, old - step)
        fm = loss(P)
        setattr(P, name, old)
        out[name] = ((fp - fm) / (2 * step), None)
    return out


def _check_fd(an, fd, rtol):
    for name, (g, idx) in fd.items():
        a = an[name]
        if idx is None:
            assert abs(a - g) <= rtol * max(1.0, abs(g)), (name, a, g)
            continue
        scale = max(1e-12, float(np.max(np.abs(a))))
        for ix in idx:
            assert abs(a[ix] - g[ix]) <= rtol * scale, (name, ix, a[ix], g[ix])


def test_pool_backward_matches_finite_differences():
    """The VJP of Eq. 5 against central differences of the (separately
    pinned) forward pool_keys, for every parameter: a dropped term or a
    transposed weight shows up as a mismatch."""
    rng = np.random.default_rng(5)
    d, h, N = 8, 16, 4
    P = O.Pooler(rng.normal(size=d) / np.sqrt(d), 0.8, 0.4, rng.normal(size=(h, 2 * d)) / np.sqrt(d),
                 rng.normal(size=h) * 0.3, rng.normal(size=(d, h)) / np.sqrt(h), 1e-6)
    X = rng.normal(size=(N, 16, d))
    dK = rng.normal(size=(N, d))
    an = O.pool_backward(X, P, dK)
    fd = _fd_grads(lambda Q: float(np.sum(dK * O.pool_keys(X, Q))), P)
    _check_fd(an, fd, 1e-6)


def test_pool_backward_of_shift_penalty_matches_finite_differences():
    """The gradient of the Eq. 7 penalty (shift_penalty_dm fed to
    pool_backward) against central differences of shift_penalty itself."""
    rng = np.random.default_rng(6)
    d, h, N = 8, 16, 6
    P = O.Pooler(rng.normal(size=d) / np.sqrt(d), 1.3, 0.5, rng.normal(size=(h, 2 * d)) / np.sqrt(d),
                 rng.normal(size=h) * 0.3, rng.normal(size=(d, h)) / np.sqrt(h), 1e-6)
    X = rng.normal(size=(N, 16, d)) + 0.5
    an = O.pool_backward(X, P, np.zeros((N, d)), O.shift_penalty_dm(X, P))
    fd = _fd_grads(lambda Q: O.shift_penalty({1: X}, Q)[1], P)
    _check_fd(an, fd, 1e-6)
    assert an["g"] == 0.0                   # the penalty does not involve g


def test_kl_key_grad_matches_finite_differences():
    """The gradient of a query's Eq. 6 terms with respect to node keys
    (exact-mode logits) against central differences of distill_kl over a
    perturbed tree, at two scored levels; the split form agrees with it to
    the float32 rounding of its operands."""
    rng = np.random.default_rng(9)
    d, C, k, L, theta = 8, 16, 3, 5000, 1e4
    P = _pooler(d, 16, 3)
    K0 = rng.normal(size=(L, d))
    K, _ = O.build_tree(K0, rng.normal(size=(L, d)), C, 4, P, "f32")
    t = L - 1
    qG = rng.normal(size=(2, d))
    tr = O.walk(qG, t, K, C, k, exact=True, theta=theta)
    assert sorted(l for l, lt in tr.levels.items() if lt.scored) == [1, 2]
    an = O.kl_key_grad(qG, t, tr, K0, C, theta, exact=True)
    step = 1e-6
    for lvl in (1, 2):
        nodes, g = an[lvl]
        for i in (0, len(nodes) // 2, len(nodes) - 1):
            u = int(nodes[i])
            for jj in (0, d - 1):
                Kp = [x.copy() for x in K]
                Km = [x.copy() for x in K]
                Kp[lvl][u, jj] += step
                Km[lvl][u, jj] -= step
                fp = sum(O.distill_kl(qG, t, O.walk(qG, t, Kp, C, k, exact=True, theta=theta),
                                      K0, C, theta).values())
                fm = sum(O.distill_kl(qG, t, O.walk(qG, t, Km, C, k, exact=True, theta=theta),
                                      K0, C, theta).values())
                fd = (fp - fm) / (2 * step)
                assert abs(g[i, jj] - fd) <= 1e-6 * max(1.0, np.abs(g).max()), (lvl, u, jj, g[i, jj], fd)
    cos, sin = O.rope_table(d, C * k, theta)
    trs = O.walk(qG, t, K, C, k, cos, sin, "f32", theta=theta)
    sp = O.kl_key_grad(qG, t, trs, K0, C, theta, cos, sin, "f32")
    for lvl in (1, 2):
        assert np.array_equal(sp[lvl][0], an[lvl][0])
        assert np.max(np.abs(sp[lvl][1] - an[lvl][1])) <= 1e-5 * np.abs(an[lvl][1]).max()
