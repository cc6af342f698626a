"""The staged GPU-vs-oracle comparison (``tests/parity.py``) checked on the
CPU: fed the oracle's own results it accepts them, and every planted mistake
in the "kernel" results -- a node off by more than its bar, a swap that is not
a near-tie, a wrong output -- is rejected, while a near-tie swap is accepted
and followed (the lower levels and the output are then still compared)."""

from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import recsa_oracle as O
from tests import parity as PY

C, K_SEL, D, G, L = 16, 16, 64, 2, 4600


def _pdict(seed):
    g = np.random.default_rng(seed)
    sd = 1.0 / np.sqrt(D)
    t = lambda *s: torch.tensor(g.normal(0.0, sd, s), dtype=torch.float32)
    return {"w": t(D), "W1": t(D, 2 * D), "b1": t(D), "W2": t(D, D), "tau": 1.0, "g": 0.5,
            "eps": 1e-6}


def _fake_tree(seed=3, zero_keys=False):
    """A float32 tree as a kernel would store it: the oracle's levels rounded
    to float32, as torch tensors [B=1][Hkv=1][rows][d].  zero_keys: all
    token keys 0 and W2 = 0, so every node key is 0 too (every logit 0)."""
    g = np.random.default_rng(seed)
    K0 = O.rnd(g.normal(size=(L, D)), "f32")
    V0 = O.rnd(g.normal(size=(L, D)), "f32")
    pd = _pdict(seed)
    if zero_keys:
        K0[:] = 0.0
        pd["W2"].zero_()
    n_lv = O.n_levels_for(L - 1, C, K_SEL)
    Kt, Vt = O.build_tree(K0, V0, C, n_lv, PY.oracle_pooler(pd), "f32")
    as_t = lambda a: torch.tensor(a, dtype=torch.float32).view(1, 1, *a.shape)
    tree = SimpleNamespace(K=[as_t(x) for x in Kt], V=[as_t(x) for x in Vt], n_levels=n_lv,
                           dtype="f32", k=K_SEL, d=D)
    return tree, pd, g


def _kernel_like(qG, t, K, V):
    """What a kernel reports for one (query, KV head), from the oracle: the
    selection [n_sel][k] (-1 padded), counts, importances [n_sel][C k] and the
    output, at the allocated level count."""
    cos, sin = O.rope_table(D, C * K_SEL, 1e6)
    n_lv = len(K)
    D_t = O.n_levels_for(t, C, K_SEL)
    Kt = [K[0][: t + 1]] + [K[l][: (t + 1) // C ** l] for l in range(1, n_lv)]
    Vt = [V[0][: t + 1]] + [V[l][: (t + 1) // C ** l] for l in range(1, n_lv)]
    o, tr = O.decode_reference(qG, t, Kt[:D_t], Vt[:D_t], C, K_SEL, cos, sin, "f32")
    sel = -np.ones((n_lv - 1, K_SEL), np.int32)
    cnt = np.zeros(n_lv - 1, np.int32)
    imp = np.zeros((n_lv - 1, C * K_SEL), np.float32)
    for lvl in range(1, n_lv):
        if lvl in tr.levels:
            S = tr.levels[lvl].S
            if tr.levels[lvl].scored:
                imp[lvl - 1, : len(tr.levels[lvl].importance)] = tr.levels[lvl].importance
        else:
            S = np.arange((t >> (4 * lvl)) + 1)
        sel[lvl - 1, : len(S)] = S
        cnt[lvl - 1] = len(S)
    return sel, cnt, imp, o, tr, (cos, sin)


def _check(tree, pd, qG, t, sel, cnt, imp, o, tol=1e-5):
    rep = PY.WalkReport()
    K, V = PY.staged_tree(tree, pd, 0, 0, t + 1)
    cos, sin = O.rope_table(D, C * K_SEL, 1e6)
    PY.check_query(qG, t, K, V, sel, cnt, imp, o, rep, "f32", K_SEL, cos, sin, tol,
                   tree.n_levels)
    return rep


def test_protocol_accepts_the_oracle_and_rejects_planted_mistakes():
    tree, pd, g = _fake_tree()
    t = L - 1
    qG = O.rnd(g.normal(size=(G, D)), "f32")
    K = [tree.K[l][0, 0].double().numpy() for l in range(tree.n_levels)]
    V = [tree.V[l][0, 0].double().numpy() for l in range(tree.n_levels)]
    sel, cnt, imp, o, tr, _ = _kernel_like(qG, t, K, V)
    rep = _check(tree, pd, qG, t, sel, cnt, imp, o)
    assert rep.compared == 1 and rep.swapped == 0 and rep.imp_levels == 2

    # a node key off by 1e-4 relative fails stage 1
    bad = SimpleNamespace(**vars(tree))
    bad.K = [x.clone() for x in tree.K]
    bad.K[1][0, 0, 7, 3] *= 1.0 + 1e-4
    with pytest.raises(AssertionError):
        PY.staged_tree(bad, pd, 0, 0, t + 1)

    # a swap of the weakest kept node for the strongest dropped one, with a
    # real importance gap, fails stage 2
    lt = tr.levels[1]
    others = lt.A[:-1]
    kept = [x for x in lt.S[:-1]]
    dropped = [x for x in others if x not in set(lt.S.tolist())]
    I = dict(zip(others.tolist(), lt.importance.tolist()))
    weakest = min(kept, key=lambda x: I[x])
    best_out = max(dropped, key=lambda x: I[x])
    assert I[weakest] - I[best_out] > 1e-5 * I[weakest]
    s2 = sel.copy()
    row = [x for x in lt.S.tolist() if x != weakest] + [best_out]
    s2[0, : len(row)] = np.sort(row)
    with pytest.raises(AssertionError, match="kernel kept"):
        _check(tree, pd, qG, t, s2, cnt, imp, o)

    # importances off by 1e-3 relative fail
    i2 = imp.copy()
    i2[0, 5] *= 1.001
    with pytest.raises(AssertionError):
        _check(tree, pd, qG, t, sel, cnt, i2, o)

    # an output off by 1e-4 of its scale fails the float32 bar
    o2 = o.copy()
    o2[1, 9] += 1e-4 * np.abs(o).max()
    with pytest.raises(AssertionError):
        _check(tree, pd, qG, t, sel, cnt, imp, o2)


def test_protocol_follows_an_accepted_near_tie():
    """With every key 0 every candidate has the same importance (an exact
    tie; the oracle keeps the lowest indices).  The "kernel" keeps the next
    level-1 candidate instead of the last one the oracle kept.  The swap is
    accepted and counted, and the walk follows it: the level-0 list and the
    output compared are those of the kernel's choice."""
    tree, pd, g = _fake_tree(5, zero_keys=True)
    t = L - 1
    qG = O.rnd(g.normal(size=(G, D)), "f32")
    K = [tree.K[l][0, 0].double().numpy() for l in range(tree.n_levels)]
    V = [tree.V[l][0, 0].double().numpy() for l in range(tree.n_levels)]
    sel, cnt, imp, o, tr, (cos, sin) = _kernel_like(qG, t, K, V)
    lt = tr.levels[1]
    assert lt.scored and np.all(lt.importance == lt.importance[0])
    A = lt.A
    last_kept, first_dropped = int(A[K_SEL - 2]), int(A[K_SEL - 1])
    assert last_kept in set(lt.S.tolist()) and first_dropped not in set(lt.S.tolist())
    row = np.sort([v for v in lt.S.tolist() if v != last_kept] + [first_dropped])
    s2 = sel.copy()
    s2[0, : len(row)] = row
    Kt = [K[0][: t + 1]] + [K[l][: (t + 1) // C ** l] for l in range(1, tree.n_levels)]
    Vt = [V[0][: t + 1]] + [V[l][: (t + 1) // C ** l] for l in range(1, tree.n_levels)]
    o_follow, trf = O.decode_reference(
        qG, t, Kt, Vt, C, K_SEL, cos, sin, "f32",
        choose=lambda lvl, oth, imp_, S: row if lvl == 1 else S)
    assert not np.array_equal(trf.A0, tr.A0)        # the level-0 list follows the swap
    rep = _check(tree, pd, qG, t, s2, cnt, imp, o_follow)
    assert rep.swapped == 1 and rep.compared == 1
    # comparing with the oracle's own output instead would have been wrong
    assert np.abs(o_follow - o).max() > 1e-3 * np.abs(o).max()
    with pytest.raises(AssertionError):
        _check(tree, pd, qG, t, s2, cnt, imp, o)
