"""Helpers for comparing the HIP path with the CPU oracle.

The oracle always computes from the seeded inputs (never from HIP outputs).
HIP outputs are only *checked*: selections must equal the oracle's, except
where the oracle's own importances of a swapped pair are within a stated
tolerance (a near-tie the float32 kernel may break the other way); below such
a swap the candidate lists differ, so lower levels and the output of that
(query, KV head) are not compared (counted as cascaded).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from oracle import recsa_oracle as O


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
class WalkReport:
    matched: int = 0            # (query, head) pairs whose selection matched fully
    swapped: int = 0            # pairs with an allowed near-tie swap
    levels_compared: int = 0
    max_imp_rel: float = 0.0
    max_out_rel: float = 0.0
    notes: list = field(default_factory=list)


def compare_walk(tr: O.WalkTrace, sel: np.ndarray, cnt: np.ndarray, imp: np.ndarray | None,
                 rep: WalkReport, tie_rel: float, row_differs=None, loose_rel: float = 0.0):
    """Compare one (query, KV head).  sel [n_sel][k], cnt [n_sel], imp
    [n_sel][C*k] (or None) are the GPU's.  Returns True when every level
    matched (so the output can be compared)."""
    for lvl in sorted(tr.levels, reverse=True):
        lt = tr.levels[lvl]
        slot = lvl - 1
        g_cnt = int(cnt[slot])
        assert g_cnt == len(lt.S), (lvl, g_cnt, len(lt.S))
        g_S = sel[slot][:g_cnt].astype(np.int64)
        assert np.all(sel[slot][g_cnt:] == -1) or g_cnt == sel.shape[1]
        rep.levels_compared += 1
        if lt.scored and imp is not None:
            n = len(lt.A) - 1
            gi = imp[slot][:n]
            rel = np.max(np.abs(gi - lt.importance) / np.maximum(lt.importance, 1e-30))
            rep.max_imp_rel = max(rep.max_imp_rel, float(rel))
        if np.array_equal(g_S, lt.S):
            continue
        assert lt.scored, f"unscored level {lvl} differs"
        others = lt.A[:-1]
        I = dict(zip(others.tolist(), lt.importance.tolist()))
        gx = sorted(set(g_S.tolist()) - set(lt.S.tolist()))
        oy = sorted(set(lt.S.tolist()) - set(g_S.tolist()))
        assert len(gx) == len(oy)
        for x in gx:
            for y in oy:
                tol = tie_rel * I[y]
                if row_differs is not None and (row_differs(lvl, x) or row_differs(lvl, y)):
                    tol = max(tol, loose_rel * I[y])
                assert I[y] - I[x] <= tol, (
                    f"level {lvl}: GPU kept {x} (I={I[x]:.9g}) over {y} (I={I[y]:.9g})")
        rep.swapped += 1
        rep.notes.append((tr.t, lvl, gx, oy))
        return False
    rep.matched += 1
    return True


def out_rel_err(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    return float(np.max(np.abs(o_gpu - o_ref)) / np.max(np.abs(o_ref)))
