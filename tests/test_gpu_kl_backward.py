"""Gradient of the Eq. 6 terms with respect to the node keys, HIP path vs the
CPU oracle through the C ABI (picx.dev Pooler Distillation, Eq. 6).

recsa_select (importances, logits kept in its workspace), recsa_distill_kl
(teacher distributions), then recsa_distill_key_grad; the oracle walks its
own trees and sums kl_key_grad (pinned by finite differences) over the same
queries.  Bar: each element within 1e-4 (float32 trees) or 2e-4 (bf16) of
the sum over its terms of their uncancelled size (the oracle's magnitude
bound: float32 logits, importances and teacher masses carry ~1e-5 relative
error, which the cancelling difference r - sum r P can amplify only up to
that size); rows no query scores are exactly 0; two calls give identical
bits.  Every compared (query, head) walk must match the oracle's selection.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import recsa_oracle as O
from tests import parity as PY
from tests import test_gpu_distill as TD

pytestmark = pytest.mark.gpu

R = pytest.importorskip("long_context_kv_amd.recsa")
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R.lib()


def run_key_grad(tree, q, Hq, pos):
    B, T = pos.shape
    nq = B * T
    ws = R.workspace(tree, Hq, nq)
    sel, cnt, imp = tree.selection_buffers(nq, with_importance=True)
    R.recsa_select(tree, q, Hq, T, pos, sel, cnt, imp, ws)
    dws = torch.empty(R.recsa_distill_workspace_bytes(tree, Hq, nq), dtype=torch.uint8, device=DEV)
    kl = torch.empty((B, T, tree.Hkv, tree.n_sel), dtype=torch.float32, device=DEV)
    y = torch.empty((nq, tree.Hkv, tree.n_sel, 16 * tree.k), dtype=torch.float32, device=DEV)
    R.recsa_distill_kl(tree, q, Hq, T, pos, sel, cnt, imp, TD.THETA, kl, dws, teacher=y)
    kws = torch.empty(R.recsa_distill_key_grad_workspace_bytes(tree, Hq, nq), dtype=torch.uint8,
                      device=DEV)
    outs = []
    for _ in range(2):
        buf, views = R.key_grad_buffer(tree)
        buf.fill_(float("nan"))
        R.recsa_distill_key_grad(tree, q, Hq, T, pos, sel, cnt, imp, y, ws, buf, kws)
        outs.append((buf, views))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])          # fixed summation order
    return (sel.cpu().numpy().reshape(B, T, tree.Hkv, tree.n_sel, tree.k),
            cnt.cpu().numpy().reshape(B, T, tree.Hkv, tree.n_sel),
            imp.cpu().numpy().reshape(B, T, tree.Hkv, tree.n_sel, -1),
            [v.cpu().numpy().astype(np.float64) for v in outs[0][1]])


@pytest.mark.parametrize("dtype,d,tol", [("f32", 64, 1e-4), ("f32", 128, 1e-4),
                                         ("bf16", 128, 2e-4)])
def test_key_grad_matches_oracle(dtype, d, tol):
    """20 queries on 2 KV heads (G = 4) of a 5000-token tree at k = 16 (levels
    1 and 2 scored), positions spread over the sequence."""
    _need_gpu()
    L0, T, k = 5000, 20, 16
    tree, pool, pdict = TD._tree(1, 2, d, L0, k, dtype, 91)
    Hq = 8
    q = synth.to_storage(synth.normal((1, T, Hq, d), DEV, 91, 1), dtype)
    pos = torch.tensor([TD.positions(L0, T, 91)], dtype=torch.int64, device=DEV)
    T = pos.shape[1]
    sel, cnt, imp, dK = run_key_grad(tree, q, Hq, pos)
    assert compare_with_oracle(tree, pdict, q, pos, sel, cnt, imp, dK, range(tree.Hkv),
                               tol) == (tree.Hkv, True)


def test_key_grad_two_sequences_and_head_ratios():
    """Two sequences (each with its own positions and chunk), G = 2 and
    G = 1, k = 64 on 9000 tokens (level 1 scored from t = 1024 on)."""
    _need_gpu()
    L0, T, k, d = 9000, 10, 64, 64
    tree, pool, pdict = TD._tree(2, 2, d, L0, k, "bf16", 92)
    for G in (2, 1):
        Hq = 2 * G
        q = synth.to_storage(synth.normal((2, T, Hq, d), DEV, 92, G), "bf16")
        pos = torch.stack([torch.tensor(TD.positions(L0, T, 92 + s)) for s in range(2)]).to(DEV)
        sel, cnt, imp, dK = run_key_grad(tree, q, Hq, pos)
        n, scored = compare_with_oracle(tree, pdict, q, pos, sel, cnt, imp, dK, range(tree.Hkv),
                                        list_bar(k))
        assert n == 2 * tree.Hkv and scored, (G, n)


def list_bar(k):
    """The bf16 bar for lists of up to 16 k candidates."""
    return tolerance(2e-4, 16 * k)


def tolerance(base, n_cand):
    """The bar for lists of up to n_cand candidates: the small cases' base
    (lists of at most 256) plus 4 n_cand 2^-24, the worst-case relative error
    of the four float32 sums over a list (the student softmax's normaliser,
    the importance's, the teacher mass's renormalisation and sum_f r_f P_f),
    which grows with the list length."""
    return base + 4.0 * max(n_cand - 256, 0) * 2.0 ** -24


def compare_with_oracle(tree, pdict, q, pos, sel, cnt, imp, dK, heads, tol):
    """The oracle's kl_key_grad summed over the queries of pos (every
    sequence), per sequence and KV head in heads, against dK to the
    magnitude-scaled bar.  The oracle walks the stored tree (checked node by
    node first) and must reach the kernel's selection, following it only at
    accepted near-ties; the importances are compared on the way.  Returns the
    number of (sequence, head) pairs compared and whether any of them had a
    scored term."""
    compared, scored = 0, False
    k, d, dtype = tree.k, tree.d, tree.dtype
    Hq = q.shape[2]
    T = pos.shape[1]
    cos, sin = O.rope_table(d, 16 * k, TD.THETA)
    qn = PY.to64(q)
    G = Hq // tree.Hkv
    rep = PY.WalkReport()
    for b in range(pos.shape[0]):
        n_tok = int(pos[b].max()) + 1
        for j in heads:
            K, V = PY.staged_tree(tree, pdict, b, j, n_tok)
            K0 = K[0]
            ref = [np.zeros_like(dK[l][b, j]) for l in range(tree.n_levels - 1)]
            mag = [np.zeros_like(dK[l][b, j]) for l in range(tree.n_levels - 1)]
            for ti in range(T):
                t = int(pos[b, ti])
                qG = qn[b, ti, j * G:(j + 1) * G]
                tr = PY.check_query(qG, t, K, V, sel[b, ti, j], cnt[b, ti, j], imp[b, ti, j],
                                    np.zeros((G, d)), rep, dtype, k, cos, sin, np.inf,
                                    tree.n_levels)
                g = O.kl_key_grad(qG, t, tr, K0[: t + 1], 16, TD.THETA, cos, sin, dtype)
                m = O.kl_key_grad(qG, t, tr, K0[: t + 1], 16, TD.THETA, cos, sin, dtype,
                                  magnitude=True)
                for lvl, (nodes, v) in g.items():
                    ref[lvl - 1][nodes] += v
                    mag[lvl - 1][nodes] += m[lvl][1]
            else:
                _check_head(tree, dK, b, j, ref, mag, tol)
                compared += 1
                scored |= any(m_.max() > 0 for m_ in mag)
    return compared, scored


def _check_head(tree, dK, b, j, ref, mag, tol):
    """Rows no query scores exactly 0, the rest within tol of their terms'
    summed magnitude."""
    for l in range(tree.n_levels - 1):
        got = dK[l][b, j]
        assert np.all(np.isfinite(got)), l
        untouched = mag[l].max(axis=1) == 0
        assert np.all(got[untouched] == 0.0), l
        err = np.abs(got - ref[l])
        assert np.all(err <= tol * mag[l] + 1e-30), \
            (b, j, l + 1, float(np.max(err / (mag[l] + 1e-30))))
