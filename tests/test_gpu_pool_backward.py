"""Pooler backward of the HIP path vs the CPU oracle, through the C ABI
(picx.dev Pooler Distillation, Eq. 5 trained with Eq. 7; Training Stages).

recsa_pooler_backward gives the gradients of sum_i dK_i . K_i + lambda *
penalty over a level's complete nodes; the oracle's pool_backward (pinned by
finite differences) gets the same seeded dK and its own shift_penalty_dm.
Bar: each gradient element within 1e-4 of the sum over nodes of the
magnitudes of its per-node terms (each term is float32 arithmetic, the sum
float64, so the error scales with that sum, not with the possibly cancelling
total); 1e-3 above level 1 of a bf16 tree, whose children are the oracle's
own level-1 keys, which may differ from the GPU's by a rounding flip.
Repeated calls are bit-identical.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import recsa_oracle as O
from tests import parity as PY

pytestmark = pytest.mark.gpu

R = pytest.importorskip("long_context_kv_amd.recsa")
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R.lib()


def gpu_backward(tree, pool, level, tok_end, dK, lam):
    """recsa_shift_penalty for the level's sums, then recsa_pooler_backward."""
    dev = tree.rope.device
    sws = torch.empty(R.recsa_shift_workspace_bytes(tree), dtype=torch.uint8, device=dev)
    pen = torch.zeros((tree.n_levels - 1, tree.d + 2), dtype=torch.float32, device=dev)
    R.recsa_shift_penalty(tree, pool, tok_end, pen, sws)
    ws = torch.empty(R.recsa_pooler_backward_workspace_bytes(tree, pool, level),
                     dtype=torch.uint8, device=dev)
    grads = []
    for _ in range(2):
        g = R.pooler_grad_buffers(pool)
        for v in g.values():
            v.fill_(float("nan"))
        R.recsa_pooler_backward(tree, pool, level, tok_end, dK,
                                pen[level - 1] if lam else None, lam, g, ws)
        grads.append(g)
    torch.cuda.synchronize()
    for n in grads[0]:
        assert torch.equal(grads[0][n], grads[1][n]), n    # fixed summation order
    return {n: v.cpu().double().numpy() for n, v in grads[0].items()}


def oracle_backward(tree, pdict, level, tok_end, dK, lam):
    """The oracle on its own trees (built from the seeded tokens): the
    children of every complete node of the level, all heads, and the
    matching dK rows."""
    P = PY.oracle_pooler(pdict)
    Xs, dKs = [], []
    n = tok_end // 16 ** level
    for b in range(tree.B):
        for j in range(tree.Hkv):
            K0 = PY.to64(tree.K[0][b, j, :tok_end])
            V0 = PY.to64(tree.V[0][b, j, :tok_end])
            K, _ = O.build_tree(K0, V0, 16, level + 1, P, tree.dtype)
            Xs.append(K[level - 1][: n * 16].reshape(n, 16, -1))
            dKs.append(np.zeros((n, tree.d)) if dK is None else PY.to64(dK[b, j, :n]))
    X, dKa = np.concatenate(Xs), np.concatenate(dKs)
    extra = lam * O.shift_penalty_dm(X, P) if lam else np.zeros_like(dKa)
    ref = O.pool_backward(X, P, dKa, extra)
    mag = None                          # sum over nodes of |per-node term|
    for i in range(X.shape[0]):
        gi = O.pool_backward(X[i:i + 1], P, dKa[i:i + 1], extra[i:i + 1])
        if mag is None:
            mag = {n: np.abs(np.asarray(v, dtype=np.float64)) for n, v in gi.items()}
        else:
            for n, v in gi.items():
                mag[n] = mag[n] + np.abs(np.asarray(v, dtype=np.float64))
    return ref, mag


def compare(g, ref_mag, tol):
    ref, mag = ref_mag
    for name in ("w", "W1", "b1", "W2", "tau", "g"):
        a = np.asarray(g[name], dtype=np.float64).reshape(np.shape(ref[name]))
        r = np.asarray(ref[name], dtype=np.float64)
        bound = tol * (np.asarray(mag[name]) + 1e-30)
        bad = np.abs(a - r) > bound
        assert not np.any(bad), (name, float(np.max(np.abs(a - r) / bound)))


@pytest.mark.parametrize("dtype,d,B,Hkv,L0,tok_end,levels,lam,with_dk", [
    ("f32", 64, 1, 1, 4096, 4096, (1, 2), 0.7, True),
    ("bf16", 128, 2, 2, 8200, 8200, (1, 2), 0.5, True),
    ("bf16", 128, 1, 2, 8200, 300, (1,), 1.0, False),     # 18 nodes: a ragged tile; penalty only
    ("f32", 128, 1, 1, 4096, 4096, (1,), 0.3, True),
    ("bf16", 64, 1, 2, 4200, 4200, (1, 2), 0.6, True),
])
def test_pooler_backward_matches_oracle(dtype, d, B, Hkv, L0, tok_end, levels, lam, with_dk):
    _need_gpu()
    wl = synth.Workload("bwd", B, Hkv, Hkv * 4, d, dtype, L0, 16, 16, 81)
    K, V = synth.kv_rows(wl, DEV, n_rows=L0)
    pdict = synth.pooler_params(d, d, DEV, 81)
    tree = R.Tree.allocate(B, Hkv, d, L0, k=16, dtype=dtype, device=DEV, level0=(K, V))
    pool = R.Pooler.from_dict(pdict, DEV)
    R.recsa_build_tree(tree, pool, 0, L0)
    for level in levels:
        rows = R.recsa_level_rows(L0, 16, level)
        dK = synth.normal((B, Hkv, rows, d), DEV, 81, level) if with_dk else None
        g = gpu_backward(tree, pool, level, tok_end, dK, lam)
        ref = oracle_backward(tree, pdict, level, tok_end, dK, lam)
        tol = 1e-3 if (dtype == "bf16" and level > 1) else 1e-4
        compare(g, ref, tol)
