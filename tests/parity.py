"""Helpers for comparing the HIP path with the CPU oracle: the staged protocol.

The oracle's own inputs are the seeded rows; every stage below takes the
HIP path's result of the stage before as its input only after that result has
itself been checked at its own bar, so that one rounding flip cannot cascade:

1. Tree.  Every stored node of level l >= 1 is recomputed by the oracle from
   the stored children the kernel read (level 0 is the seeded input itself)
   and must match within one storage ulp, plus the float32 evaluation error
   relative to the row's scale (a near-zero entry of a node key is a
   cancellation of terms of the row's size).
2. Selection.  The oracle walks the stored tree.  Selected sets must be
   identical; a swapped pair is accepted only where the oracle's importances
   of the two nodes differ by less than 1e-5 relative, and the walk then
   follows the kernel's choice into the levels below (``walk(choose=...)``),
   so the lower levels and the output are still compared.  Importances, where
   the kernel reports them, are compared at every scored level.
3. Output.  The oracle attends with the stored tree and the (followed)
   selection: max relative error <= 2e-3 (bf16) or 1e-5 (float32).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from oracle import recsa_oracle as O

# Stage bars (float32 arithmetic error relative to a row's largest entry)
KEY_F32_REL = 1e-5        # float32 tree: relative to the entry ...
KEY_F32_ROW = 1e-6        # ... plus this much of the row's scale
VAL_ROW = 1e-6            # node value: mean of 16 children in float32
KEY_BF16_ROW = 4e-6       # node key: sums of C*d and hidden terms in float32
IMP_REL = 1e-4            # importance: relative ...
IMP_ABS = 1e-12           # ... with a floor for entries that underflow float32
TIE_REL = 1e-5            # accepted near-tie of a swapped pair
_TINY = np.finfo(np.float64).tiny


def to64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def oracle_pooler(p: dict) -> O.Pooler:
    f = lambda x: x.detach().cpu().double().numpy() if torch.is_tensor(x) else x
    return O.Pooler(f(p["w"]), float(p["tau"]), float(p["g"]), f(p["W1"]), f(p["b1"]),
                    f(p["W2"]), float(p.get("eps", 1e-6)))


def ulp_bf16(x):
    """Spacing of bfloat16 numbers at |x| (float64 array)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


@dataclass
class TreeReport:
    levels: int = 0
    nodes: int = 0
    key_flips: int = 0          # entries that differ from the oracle's rounding
    val_flips: int = 0
    entries: int = 0
    max_key_ratio: float = 0.0  # largest |difference| / bar


def staged_tree(tree, pdict, b: int, j: int, n_tokens: int, rep: TreeReport | None = None):
    """Stage 1 for sequence b, KV head j: check every stored node whose
    subtree lies in [0, n_tokens) against the oracle's Eq. 5 key and Eq. 1
    value computed from the stored children, then return the stored levels
    (float64) truncated to those nodes: K, V lists for the oracle's walk."""
    P = oracle_pooler(pdict)
    dt = tree.dtype
    K = [to64(tree.K[0][b, j, :n_tokens])]
    V = [to64(tree.V[0][b, j, :n_tokens])]
    for lvl in range(1, tree.n_levels):
        n = n_tokens // 16 ** lvl
        gk = to64(tree.K[lvl][b, j, :n])
        gv = to64(tree.V[lvl][b, j, :n])
        if n:
            d = gk.shape[1]
            kc = K[lvl - 1][: n * 16].reshape(n, 16, d)
            vc = V[lvl - 1][: n * 16].reshape(n, 16, d)
            rk = O.rnd(O.pool_keys(kc, P), dt)
            rv = O.rnd(O.mean_values(vc), dt)
            ks = np.abs(rk).max(axis=1, keepdims=True)
            vs = np.abs(rv).max(axis=1, keepdims=True)
            if dt == "f32":
                kb = KEY_F32_REL * np.abs(rk) + KEY_F32_ROW * ks
                vb = KEY_F32_REL * np.abs(rv) + VAL_ROW * vs
            else:
                kb = ulp_bf16(rk) + KEY_BF16_ROW * ks
                vb = ulp_bf16(rv) + VAL_ROW * vs
            kb, vb = kb + _TINY, vb + _TINY         # an all-zero row must match exactly
            dk, dv = np.abs(gk - rk), np.abs(gv - rv)
            ratio = float((dk / kb).max())
            assert np.all(dk <= kb), (b, j, lvl, "key", ratio)
            assert np.all(dv <= vb), (b, j, lvl, "value", float((dv / vb).max()))
            if rep is not None:
                rep.levels += 1
                rep.nodes += n
                rep.entries += dk.size
                rep.key_flips += int(np.count_nonzero(dk))
                rep.val_flips += int(np.count_nonzero(dv))
                rep.max_key_ratio = max(rep.max_key_ratio, ratio)
        K.append(gk)
        V.append(gv)
    return K, V


@dataclass
class WalkReport:
    compared: int = 0           # (query, KV head) pairs checked through the output
    swapped: int = 0            # accepted near-tie swaps (the walk followed the kernel)
    levels_compared: int = 0
    imp_levels: int = 0         # scored levels whose importances were compared
    max_imp_rel: float = 0.0
    max_out_rel: float = 0.0
    notes: list = field(default_factory=list)


class Follow:
    """``choose`` hook for the oracle's walk: at each scored level, accept the
    kernel's selection if it equals the oracle's, or if every swapped pair is
    a near-tie of the oracle's importances (< TIE_REL relative), and continue
    with it; otherwise fail."""

    def __init__(self, sel: np.ndarray, cnt: np.ndarray, rep: WalkReport, t: int,
                 tie_rel: float = TIE_REL):
        self.sel, self.cnt, self.rep, self.t, self.tie_rel = sel, cnt, rep, t, tie_rel

    def __call__(self, lvl, others, I, S):
        g_cnt = int(self.cnt[lvl - 1])
        g_S = np.sort(self.sel[lvl - 1][:g_cnt].astype(np.int64))
        if np.array_equal(g_S, S):
            return S
        assert len(g_S) == len(S), (self.t, lvl, len(g_S), len(S))
        imp = dict(zip(others.tolist(), np.asarray(I).tolist()))
        gx = sorted(set(g_S.tolist()) - set(S.tolist()))    # kernel kept, oracle dropped
        oy = sorted(set(S.tolist()) - set(g_S.tolist()))    # oracle kept, kernel dropped
        assert S[-1] in set(g_S.tolist()), (self.t, lvl, "current node dropped")
        for x in gx:
            assert x in imp, (self.t, lvl, f"kernel kept {x}, not a candidate")
            for y in oy:
                assert imp[y] - imp[x] <= self.tie_rel * imp[y], (
                    f"t={self.t} level {lvl}: kernel kept {x} (I={imp[x]:.9g}) "
                    f"over {y} (I={imp[y]:.9g})")
        self.rep.swapped += 1
        self.rep.notes.append((self.t, lvl, gx, oy))
        return g_S


def check_query(qG, t: int, K, V, sel, cnt, imp, out, rep: WalkReport, dtype: str, k: int,
                cos, sin, out_tol: float, n_levels_alloc: int):
    """Stages 2 and 3 for one (query, KV head): qG [G, d] float64; K, V the
    stored levels (``staged_tree``); sel [n_sel][k], cnt [n_sel], imp
    [n_sel][C*k] or None, out [G, d] from the kernel."""
    D = O.n_levels_for(t, 16, k)
    Kt = [K[0][: t + 1]] + [K[lvl][: (t + 1) // 16 ** lvl] for lvl in range(1, len(K))]
    Vt = [V[0][: t + 1]] + [V[lvl][: (t + 1) // 16 ** lvl] for lvl in range(1, len(V))]
    Kt, Vt = Kt[: max(D, 1)], Vt[: max(D, 1)]
    follow = Follow(sel, cnt, rep, t)
    o_ref, tr = O.decode_reference(qG, t, Kt, Vt, 16, k, cos, sin, dtype, choose=follow)
    for lvl in sorted(tr.levels, reverse=True):
        lt = tr.levels[lvl]
        g_cnt = int(cnt[lvl - 1])
        assert g_cnt == len(lt.S), (t, lvl, g_cnt, len(lt.S))
        assert np.array_equal(sel[lvl - 1][:g_cnt].astype(np.int64), lt.S), (t, lvl)
        assert np.all(sel[lvl - 1][g_cnt:] == -1) or g_cnt == sel.shape[1], (t, lvl)
        rep.levels_compared += 1
        if lt.scored and imp is not None:
            n = len(lt.A) - 1
            gi = imp[lvl - 1][:n].astype(np.float64)
            di = np.abs(gi - lt.importance)
            assert np.all(di <= IMP_REL * lt.importance + IMP_ABS), (
                t, lvl, float((di / (lt.importance + IMP_ABS)).max()))
            assert np.all(imp[lvl - 1][n:] == 0.0), (t, lvl)
            rep.imp_levels += 1
            rep.max_imp_rel = max(rep.max_imp_rel, float(
                np.max(di / np.maximum(lt.importance, IMP_ABS / IMP_REL))))
    # levels above the oracle's top hold fully selected prefixes [0 .. a]
    for lvl in range(D, n_levels_alloc):
        a = t >> (4 * lvl)
        assert cnt[lvl - 1] == a + 1, (t, lvl)
        assert np.array_equal(sel[lvl - 1][: a + 1], np.arange(a + 1)), (t, lvl)
    err = out_rel_err(out, o_ref)
    rep.max_out_rel = max(rep.max_out_rel, err)
    assert err <= out_tol, (t, err)
    rep.compared += 1
    return tr


def out_rel_err(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    return float(np.max(np.abs(o_gpu - o_ref)) / np.max(np.abs(o_ref)))
