"""HIP path vs the CPU oracle, element by element, through the C ABI, with
the staged protocol of ``tests/parity.py``: tree nodes within one storage ulp
of the oracle's node from the same stored children (float32: 1e-5 relative);
selections equal, except near-ties where the oracle's importances of the
swapped pair differ by less than 1e-5 relative, after which the oracle follows
the kernel's choice; importances within 1e-4 relative; outputs within 1e-5
(float32) or 2e-3 (bfloat16) max relative error.
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


def _setup(B, Hkv, d, L_tokens, L_cap, k, dtype, seed, hidden=None):
    """Seeded level-0 rows [B, Hkv, L_cap, d] (first L_tokens filled), pooler."""
    wl = synth.Workload("t", B, Hkv, Hkv * 4, d, dtype, L_tokens, 16, k, seed)
    K, V = synth.kv_rows(wl, DEV, n_rows=L_cap)
    pdict = synth.pooler_params(d, hidden or d, DEV, seed)
    tree = R.Tree.allocate(B, Hkv, d, L_cap, k=k, dtype=dtype, device=DEV, level0=(K, V))
    pool = R.Pooler.from_dict(pdict, DEV)
    return wl, tree, pool, pdict


# ---------------------------------------------------------------------------

def test_rope_table_matches_oracle():
    _need_gpu()
    for d, n in ((64, 256), (128, 4096)):
        t = torch.empty((n, d // 2, 2), dtype=torch.float32, device=DEV)
        R.recsa_init_rope(t, d, n, 1e6)
        torch.cuda.synchronize()
        cos, sin = O.rope_table(d, n, 1e6)
        g = t.cpu().numpy()
        diff = np.maximum(np.abs(g[..., 0] - cos), np.abs(g[..., 1] - sin))
        assert diff.max() <= 2.0 ** -24, diff.max()
        assert (diff > 0).mean() < 1e-4


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("f32", 128), ("bf16", 64)])
def test_build_tree_matches_oracle(dtype, d):
    """Stage 1 of the parity protocol on a 3-level tree with a ragged tail:
    every stored node equals the oracle's node computed from its stored
    children (level 1 from the seeded tokens) within one storage ulp plus the
    float32 evaluation error; incomplete nodes stay unbuilt."""
    _need_gpu()
    L = 16 ** 3 * 2 + 37                     # ragged tail: incomplete nodes stay unbuilt
    wl, tree, pool, pdict = _setup(1, 2, d, L, L, 16, dtype, 11)
    R.recsa_build_tree(tree, pool, 0, L)
    torch.cuda.synchronize()
    rep = PY.TreeReport()
    for j in range(2):
        PY.staged_tree(tree, pdict, 0, j, L, rep)
        for lvl in range(1, tree.n_levels):
            assert tree.K[lvl].shape[2] == L // 16 ** lvl
    assert rep.levels == 2 * (tree.n_levels - 1)
    # rounding flips (float32 result on the other side of a bf16 rounding
    # boundary from the exact value) are rare
    assert rep.key_flips <= (2e-3 if dtype == "bf16" else 1.0) * rep.entries, rep
    print(f"  tree: {rep.nodes} nodes, key entries off the oracle's rounding "
          f"{rep.key_flips}/{rep.entries}, values {rep.val_flips}, worst/bar {rep.max_key_ratio:.2f}")
    _check_rotated_keys(tree, [(0, j) for j in range(2)], L)


def _check_rotated_keys(tree, heads, n_tokens):
    """Kr[l][i] must be the key half of the split RoPE of the stored key row,
    rnd(R(i mod 16) K[l][i]), evaluated as the oracle evaluates it (float32
    rotation, rounded to the storage dtype).  Equal except where the two
    RoPE tables differ in a float32 ulp (rare), and then by at most one ulp."""
    if tree.Kr[0].numel() == 0:
        return                                    # a tree without the rotated-key copy
    cos, sin = O.rope_table(tree.d, tree.C * tree.k, 1e6)
    for b, j in heads:
        for lvl in range(tree.n_levels):
            n = n_tokens // 16 ** lvl
            if n == 0:
                continue
            K = PY.to64(tree.K[lvl][b, j, :n])
            c = np.arange(n) % 16
            want = O.rnd(O.rotate_f32(K, cos[c], sin[c]).astype(np.float64), tree.dtype)
            got = PY.to64(tree.Kr[lvl][b, j, :n])
            diff = np.abs(got - want)
            ulp = PY.ulp_bf16(want) if tree.dtype == "bf16" else np.abs(want) * 2.0 ** -23 + 1e-38
            assert np.all(diff <= ulp), (lvl, float((diff / ulp).max()))
            assert (diff > 0).mean() < 1e-3, (lvl, (diff > 0).mean())


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("f32", 128), ("bf16", 64)])
def test_append_equals_build(dtype, d):
    """Appending tokens one at a time (completing nodes on the fly) gives
    exactly the tree a single build gives."""
    _need_gpu()
    L0, n_app = 4096 - 40, 300
    L_cap = L0 + n_app
    wl, tree, pool, pdict = _setup(2, 2, d, L_cap, L_cap, 16, dtype, 12)
    ref = R.Tree.allocate(2, 2, d, L_cap, k=16, dtype=dtype, device=DEV,
                          level0=(tree.K[0].clone(), tree.V[0].clone()))
    R.recsa_build_tree(ref, pool, 0, L_cap)
    # the appending tree starts from a build of [0, L0) and fresh rows after
    newk, newv = tree.K[0][:, :, L0:].clone(), tree.V[0][:, :, L0:].clone()
    tree.K[0][:, :, L0:] = 0
    tree.V[0][:, :, L0:] = 0
    R.recsa_build_tree(tree, pool, 0, L0)
    for i in range(n_app):
        pos = torch.full((2,), L0 + i, dtype=torch.int64, device=DEV)
        R.recsa_append_decode(tree, pool, newk[:, :, i].contiguous(), newv[:, :, i].contiguous(), pos)
    torch.cuda.synchronize()
    for lvl in range(tree.n_levels):
        assert torch.equal(tree.K[lvl], ref.K[lvl]), lvl
        assert torch.equal(tree.V[lvl], ref.V[lvl]), lvl
        assert torch.equal(tree.Kr[lvl], ref.Kr[lvl]), lvl


def _run_select_attn(tree, q, Hq, pos, decode):
    B, T = pos.shape
    nq = B * T
    ws = R.workspace(tree, Hq, nq)
    sel, cnt, imp = tree.selection_buffers(nq, with_importance=True)
    R.recsa_select(tree, q, Hq, T, pos, sel, cnt, imp, ws)
    out = torch.empty((B, T, Hq, tree.d), dtype=torch.float32, device=DEV)
    if decode:
        assert T == 1
        R.recsa_attn_decode(tree, q, Hq, pos, sel, cnt, out, ws)
    else:
        R.recsa_attn_prefill(tree, q, Hq, T, pos, sel, cnt, out, ws)
    torch.cuda.synchronize()
    return (sel.cpu().numpy().reshape(B, T, tree.Hkv, tree.n_sel, tree.k),
            cnt.cpu().numpy().reshape(B, T, tree.Hkv, tree.n_sel),
            imp.cpu().numpy().reshape(B, T, tree.Hkv, tree.n_sel, -1),
            out.cpu().numpy().astype(np.float64))


def _check_queries(tree, pdict, q, pos, sel, cnt, imp, out, heads, out_tol, trees=None,
                   seqs=None):
    """The staged protocol (``tests/parity.py``) for every (b, query, KV head
    in `heads`): stage 1 checks the stored tree of each (sequence, head) once
    (cached in `trees`), then the oracle walks it, following the kernel's
    choice at accepted near-ties, and the selection, importances (where
    given) and output are compared.  seqs[b] is the tree's sequence index of
    row b of the arrays (default b)."""
    B, T = pos.shape
    G = q.shape[2] // tree.Hkv
    cos, sin = O.rope_table(tree.d, tree.C * tree.k, 1e6)
    rep = PY.WalkReport()
    rep.tree = PY.TreeReport()
    qn = PY.to64(q)
    trees = trees if trees is not None else {}
    for b in range(B):
        sb = b if seqs is None else seqs[b]
        n_tok = int(pos[b].max()) + 1
        for j in heads:
            if (sb, j) not in trees or trees[(sb, j)][0] < n_tok:
                trees[(sb, j)] = (n_tok, PY.staged_tree(tree, pdict, sb, j, n_tok, rep.tree))
            K, V = trees[(sb, j)][1]
            for ti in range(T):
                PY.check_query(qn[b, ti, j * G:(j + 1) * G], int(pos[b, ti]), K, V,
                               sel[b, ti, j], cnt[b, ti, j],
                               None if imp is None else imp[b, ti, j],
                               out[b, ti, j * G:(j + 1) * G], rep, tree.dtype, tree.k, cos, sin,
                               out_tol, tree.n_levels)
    print(f"  parity: {rep.compared} (query, head) pairs, {rep.swapped} near-tie swaps "
          f"followed, {rep.imp_levels} importance levels (max rel {rep.max_imp_rel:.2e}), "
          f"max out rel {rep.max_out_rel:.2e}; tree flips {rep.tree.key_flips}/"
          f"{rep.tree.entries}", flush=True)
    return rep


def test_tiny_fp32_decode_queries():
    """Tiny workload: 1 KV head, 4 query heads, d=64, fp32, L=4096, k=16 (3
    levels); 8 queries at the last positions, through the T-query path and
    each through the decode path (split + combine)."""
    _need_gpu()
    wl = synth.WORKLOADS["tiny"]
    K, V = synth.kv_rows(wl, DEV)
    pdict = synth.pooler_params(wl.d, wl.d, DEV, wl.seed)
    tree = R.Tree.allocate(1, 1, wl.d, wl.L, k=wl.k, dtype="f32", device=DEV, level0=(K, V))
    assert tree.n_levels == 3
    pool = R.Pooler.from_dict(pdict, DEV)
    R.recsa_build_tree(tree, pool, 0, wl.L)
    q = synth.decode_queries(wl, DEV)                       # [1, 8, 4, 64]
    pos = torch.arange(wl.L - 8, wl.L, device=DEV).view(1, 8)
    sel, cnt, imp, out = _run_select_attn(tree, q, wl.Hq, pos, decode=False)
    trees = {}
    rep = _check_queries(tree, pdict, q, pos.cpu(), sel, cnt, imp, out, [0], 1e-5, trees)
    assert rep.compared == 8 and rep.imp_levels >= 8, rep
    for i in range(8):
        qi = q[:, i:i + 1].contiguous()
        pi = pos[:, i:i + 1].contiguous()
        s2, c2, m2, o2 = _run_select_attn(tree, qi, wl.Hq, pi, decode=True)
        assert np.array_equal(s2[0, 0], sel[0, i]) and np.array_equal(c2[0, 0], cnt[0, i])
        assert np.allclose(o2[0, 0], out[0, i], rtol=0, atol=1e-6 * np.abs(out[0, i]).max())


def test_edge_positions_fp32():
    """Queries at every kind of position in one call: the first token, dense
    short contexts (t < C*k), exact powers of 16, node boundaries and a
    ragged end; T-query path and decode path."""
    _need_gpu()
    L = 5000
    wl, tree, pool, pdict = _setup(1, 1, 64, L, L, 16, "f32", 13)
    R.recsa_build_tree(tree, pool, 0, L)
    ts = [0, 1, 2, 15, 16, 17, 255, 256, 257, 300, 4095, 4096, 4097, 4111, 4112, 4999]
    pos = torch.tensor([ts], dtype=torch.int64, device=DEV)
    q = synth.to_storage(synth.normal((1, len(ts), 4, 64), DEV, 13, 99), "f32")
    sel, cnt, imp, out = _run_select_attn(tree, q, 4, pos, decode=False)
    rep = _check_queries(tree, pdict, q, pos.cpu(), sel, cnt, imp, out, [0], 1e-5)
    assert rep.compared == len(ts)
    for i in (0, 5, 12, 15):
        s2, c2, m2, o2 = _run_select_attn(tree, q[:, i:i + 1].contiguous(),
                                          4, pos[:, i:i + 1].contiguous(), decode=True)
        assert np.allclose(o2[0, 0], out[0, i], rtol=0, atol=1e-6 * np.abs(out[0, i]).max())


@pytest.mark.parametrize("dtype,d,G", [("bf16", 64, 1), ("f32", 128, 2), ("bf16", 128, 1)])
def test_head_ratios_prefill_and_decode_vs_oracle(dtype, d, G):
    """G = 1 and G = 2 query heads per KV head (two KV heads, k = 16, 5000
    tokens): every query of a T-query call and a few through the decode path,
    selections and outputs against the oracle."""
    _need_gpu()
    L, Hkv, k = 5000, 2, 16
    wl, tree, pool, pdict = _setup(1, Hkv, d, L, L, k, dtype, 21)
    R.recsa_build_tree(tree, pool, 0, L)
    Hq = Hkv * G
    ts = [0, 17, 255, 256, 300, 1234, 4095, 4096, 4111, 4999]
    pos = torch.tensor([ts], dtype=torch.int64, device=DEV)
    q = synth.to_storage(synth.normal((1, len(ts), Hq, d), DEV, 21, 10 + G), dtype)
    tol = 1e-5 if dtype == "f32" else 2e-3
    sel, cnt, imp, out = _run_select_attn(tree, q, Hq, pos, decode=False)
    rep = _check_queries(tree, pdict, q, pos.cpu(), sel, cnt, imp, out, range(Hkv), tol)
    assert rep.compared == Hkv * len(ts), rep
    for i in (0, 4, len(ts) - 1):
        s2, c2, m2, o2 = _run_select_attn(tree, q[:, i:i + 1].contiguous(), Hq,
                                          pos[:, i:i + 1].contiguous(), decode=True)
        assert np.array_equal(s2[0, 0], sel[0, i]) and np.array_equal(c2[0, 0], cnt[0, i])
        assert np.allclose(o2[0, 0], out[0, i], rtol=0, atol=1e-5 * np.abs(out[0, i]).max())


def test_qwen_shape_bf16_decode_64k():
    """8 KV heads, 32 query heads, d=128, bf16, k=256 at L=65536: append the
    decode token at t=L, select, attend (decode path); every head vs oracle."""
    _need_gpu()
    L = 65536
    L_cap = L + 64
    wl, tree, pool, pdict = _setup(1, 8, 128, L + 1, L_cap, 256, "bf16", 14)
    newk = tree.K[0][:, :, L].clone()
    newv = tree.V[0][:, :, L].clone()
    R.recsa_build_tree(tree, pool, 0, L)
    pos1 = torch.tensor([L], dtype=torch.int64, device=DEV)
    R.recsa_append_decode(tree, pool, newk.contiguous(), newv.contiguous(), pos1)
    q = synth.to_storage(synth.normal((1, 1, 32, 128), DEV, 14, 98), "bf16")
    sel, cnt, imp, out = _run_select_attn(tree, q, 32, pos1.view(1, 1), decode=True)
    rep = _check_queries(tree, pdict, q, pos1.view(1, 1).cpu(), sel, cnt, imp, out,
                         range(8), 2e-3)
    assert rep.compared == 8 and rep.imp_levels == 8 * 2, rep


def test_prefill_chunk_bf16_causal():
    """A 512-query prefill chunk appended at [L0, L0+512): incremental build,
    T-query selection and attention; sampled queries vs oracle on two KV heads,
    and the last query's decode path equals its prefill result."""
    _need_gpu()
    L0, T = 20000, 512
    L_cap = L0 + T
    wl, tree, pool, pdict = _setup(1, 4, 128, L_cap, L_cap, 256, "bf16", 15)
    R.recsa_build_tree(tree, pool, 0, L0)
    R.recsa_build_tree(tree, pool, L0, L0 + T)               # the chunk's nodes
    q = synth.to_storage(synth.normal((1, T, 16, 128), DEV, 15, 97), "bf16")
    pos = torch.arange(L0, L0 + T, device=DEV).view(1, T)
    sel, cnt, imp, out = _run_select_attn(tree, q, 16, pos, decode=False)
    idx = list(range(0, T, 37)) + [T - 1]
    rep = _check_queries(tree, pdict, q[:, idx], pos[:, idx].cpu(), sel[:, idx], cnt[:, idx],
                         imp[:, idx], out[:, idx], [0, 3], 2e-3)
    assert rep.compared == 2 * len(idx) and rep.imp_levels == 2 * len(idx), rep   # level 1 scored
    s2, c2, m2, o2 = _run_select_attn(tree, q[:, T - 1:].contiguous(), 16,
                                      pos[:, T - 1:].contiguous(), decode=True)
    assert np.array_equal(s2[0, 0], sel[0, T - 1]) and np.array_equal(c2[0, 0], cnt[0, T - 1])
    assert np.allclose(o2[0, 0], out[0, T - 1], rtol=0, atol=1e-5 * np.abs(out[0, T - 1]).max())


def _fused_step(tree, pool, k_new, v_new, q, Hq, pos, ws=None):
    B = tree.B
    ws = ws if ws is not None else R.workspace(tree, Hq, B)
    sel, cnt, _ = tree.selection_buffers(B)
    out = torch.empty((B, Hq, tree.d), dtype=torch.float32, device=DEV)
    R.recsa_decode(tree, pool, k_new, v_new, q, Hq, pos, sel, cnt, out, ws)
    return sel, cnt, out, ws


def test_fused_decode_graph_replays_match_eager():
    """recsa_decode captured in a HIP graph and replayed: each replay starts
    its workgroups at another XCD than a direct launch does, so the groups'
    placement differs, yet every replay -- synchronised or back to back, with
    eager library and torch work in between -- gives the eager call's bits,
    raises no error word and leaves the control block zero."""
    _need_gpu()
    L0, B, Hkv, G, d, k = 40000, 2, 4, 4, 128, 64
    wl, tree, pool, pdict = _setup(B, Hkv, d, L0 + 64, L0 + 64, k, "bf16", 33)
    R.recsa_build_tree(tree, pool, 0, L0)
    Hq = Hkv * G
    t = L0 - 5
    kn = tree.K[0][:, :, t].clone().contiguous()
    vn = tree.V[0][:, :, t].clone().contiguous()
    q = synth.to_storage(synth.normal((B, 1, Hq, d), DEV, 33, 3), "bf16")
    pos = torch.full((B,), t, dtype=torch.int64, device=DEV)
    ws = R.workspace(tree, Hq, B)
    sel, cnt, _ = tree.selection_buffers(B)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    step = lambda: R.recsa_decode(tree, pool, kn, vn, q, Hq, pos, sel, cnt, out, ws)
    step()
    torch.cuda.synchronize()
    ref_o, ref_s = out.clone(), sel.clone()
    assert torch.isfinite(ref_o).all()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    ctl = R.decode_control_words(ws, tree, Hq)
    # the selection of a different query through the split calls between replays
    ws2 = R.workspace(tree, Hq, B)
    s2, c2, _ = tree.selection_buffers(B)
    q2 = synth.to_storage(synth.normal((B, 1, Hq, d), DEV, 33, 4), "bf16")
    for i in range(6):
        out.fill_(0.0)
        graph.replay()
        R.recsa_select(tree, q2, Hq, 1, pos.view(B, 1), s2, c2, None, ws2)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), i
        assert torch.equal(sel, ref_s), i
        assert torch.count_nonzero(ctl).item() == 0, (i, ctl[:, :4].tolist())
    for i in range(20):                            # back to back
        graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o)
    assert torch.count_nonzero(ctl).item() == 0


@pytest.mark.parametrize("dtype,d,Hkv,G,B", [("bf16", 128, 8, 4, 1), ("f32", 64, 2, 4, 2),
                                             ("bf16", 128, 4, 2, 3), ("bf16", 64, 2, 1, 2),
                                             ("f32", 128, 2, 2, 1)])
def test_fused_decode_matches_separate_calls(dtype, d, Hkv, G, B):
    """recsa_decode (append + select + attend in one launch) gives the same
    selection and output as recsa_append_decode + recsa_select +
    recsa_attn_decode, over consecutive steps that complete level-1 and
    level-2 nodes, and leaves its control words clear."""
    _need_gpu()
    L0, steps = 65536 - 3, 5                     # t = 65533 .. 65537 crosses 65536
    L_cap = L0 + 64
    Hq = Hkv * G
    wl, tree, pool, pdict = _setup(B, Hkv, d, L_cap, L_cap, 256, dtype, 21)
    ref = R.Tree.allocate(B, Hkv, d, L_cap, k=256, dtype=dtype, device=DEV,
                          level0=(tree.K[0].clone(), tree.V[0].clone()))
    rows_k = tree.K[0][:, :, L0:L0 + steps].clone()
    rows_v = tree.V[0][:, :, L0:L0 + steps].clone()
    R.recsa_build_tree(tree, pool, 0, L0)
    R.recsa_build_tree(ref, pool, 0, L0)
    ws = R.workspace(tree, Hq, B)
    ws_ref = R.workspace(ref, Hq, B)
    for i in range(steps):
        t = L0 + i
        pos = torch.full((B,), t, dtype=torch.int64, device=DEV)
        q = synth.to_storage(synth.normal((B, 1, Hq, d), DEV, 21, 500 + i), dtype)
        kn, vn = rows_k[:, :, i].contiguous(), rows_v[:, :, i].contiguous()
        sel, cnt, out, ws = _fused_step(tree, pool, kn, vn, q, Hq, pos, ws)
        R.recsa_append_decode(ref, pool, kn, vn, pos)
        s2, c2, m2, o2 = _run_select_attn(ref, q, Hq, pos.view(B, 1), decode=True)
        torch.cuda.synchronize()
        assert torch.equal(R.decode_error_words(ws, tree, Hq), torch.zeros_like(R.decode_error_words(ws, tree, Hq)))
        assert np.array_equal(sel.cpu().numpy().reshape(s2.shape), s2), t
        assert np.array_equal(cnt.cpu().numpy().reshape(c2.shape), c2), t
        o = out.cpu().numpy().astype(np.float64).reshape(o2.shape)
        assert np.allclose(o, o2, rtol=0, atol=1e-5 * np.abs(o2).max()), t
    for lvl in range(tree.n_levels):
        assert torch.equal(tree.K[lvl], ref.K[lvl]) and torch.equal(tree.V[lvl], ref.V[lvl]), lvl
        assert torch.equal(tree.Kr[lvl], ref.Kr[lvl]), lvl
    # control block: every arrival flag back at zero, no error word set
    assert torch.count_nonzero(R.decode_control_words(ws, tree, Hq).cpu()) == 0


def test_fused_decode_vs_oracle_bf16():
    """The fused decode step at the Qwen shape (8/32/128, bf16, k=256) on a
    64K-token cache: every KV head's selection and output vs the oracle."""
    _need_gpu()
    L = 65536 + 15                              # t + 1 = 65552: completes a level-1 node
    L_cap = L + 64
    wl, tree, pool, pdict = _setup(1, 8, 128, L + 1, L_cap, 256, "bf16", 22)
    kn, vn = tree.K[0][:, :, L].clone().contiguous(), tree.V[0][:, :, L].clone().contiguous()
    R.recsa_build_tree(tree, pool, 0, L)
    pos = torch.tensor([L], dtype=torch.int64, device=DEV)
    q = synth.to_storage(synth.normal((1, 1, 32, 128), DEV, 22, 98), "bf16")
    sel, cnt, out, ws = _fused_step(tree, pool, kn, vn, q, 32, pos)
    torch.cuda.synchronize()
    B, n_sel, k = 1, tree.n_sel, tree.k
    s = sel.cpu().numpy().reshape(B, 1, 8, n_sel, k)
    c = cnt.cpu().numpy().reshape(B, 1, 8, n_sel)
    imp = np.zeros((B, 1, 8, n_sel, 16 * k))
    o = out.cpu().numpy().astype(np.float64).reshape(B, 1, 32, 128)
    rep = _check_queries(tree, pdict, q, pos.view(1, 1).cpu(), s, c, None, o, range(8),
                         2e-3)
    assert rep.compared == 8, rep


@pytest.mark.parametrize("k", [64, 16])
def test_small_k_decode_and_prefill(k):
    """Selection depths below 256: the pages' k = 64 variant (C*k = 1024
    positions) and k = 16, both 4 levels at 40K tokens -- the fused decode,
    the separate decode calls and a causal prefill chunk, sampled queries and
    heads vs the oracle.  (The fused kernel keeps S^(l) in LDS at stride k,
    the stride the list of the level below reads it with.)"""
    _need_gpu()
    L0, T = 40000, 256
    L_cap = L0 + T + 64
    wl, tree, pool, pdict = _setup(1, 4, 128, L_cap, L_cap, k, "bf16", 31)
    assert tree.n_levels == 4
    R.recsa_build_tree(tree, pool, 0, L0)
    R.recsa_build_tree(tree, pool, L0, L0 + T)
    q = synth.to_storage(synth.normal((1, T, 16, 128), DEV, 31, 97), "bf16")
    pos = torch.arange(L0, L0 + T, device=DEV).view(1, T)
    sel, cnt, imp, out = _run_select_attn(tree, q, 16, pos, decode=False)
    idx = [0, 100, T - 1]
    rep = _check_queries(tree, pdict, q[:, idx], pos[:, idx].cpu(), sel[:, idx], cnt[:, idx],
                         imp[:, idx], out[:, idx], [1, 2], 2e-3)
    assert rep.compared == 2 * len(idx) and rep.imp_levels > 0, rep
    # decode at t = L0 + T: fused and separate calls agree with each other and the oracle
    t = L0 + T
    kn, vn = tree.K[0][:, :, t].clone().contiguous(), tree.V[0][:, :, t].clone().contiguous()
    qd = synth.to_storage(synth.normal((1, 1, 16, 128), DEV, 31, 98), "bf16")
    p1 = torch.tensor([t], dtype=torch.int64, device=DEV)
    ref = R.Tree.allocate(1, 4, 128, L_cap, k=k, dtype="bf16", device=DEV,
                          level0=(tree.K[0].clone(), tree.V[0].clone()))
    R.recsa_build_tree(ref, pool, 0, L0 + T)
    fs, fc, fo, ws = _fused_step(tree, pool, kn, vn, qd, 16, p1)
    R.recsa_append_decode(ref, pool, kn, vn, p1)
    s2, c2, m2, o2 = _run_select_attn(ref, qd, 16, p1.view(1, 1), decode=True)
    torch.cuda.synchronize()
    assert np.array_equal(fs.cpu().numpy().reshape(s2.shape), s2)
    assert np.allclose(fo.cpu().numpy().astype(np.float64).reshape(o2.shape), o2, rtol=0,
                       atol=1e-5 * np.abs(o2).max())
    rep2 = _check_queries(ref, pdict, qd, p1.view(1, 1).cpu(), s2, c2, m2, o2, [0, 3], 2e-3)
    assert rep2.compared == 2 and rep2.imp_levels > 0, rep2


def test_prefill_two_sequences_bucketed_matches_per_query():
    """Two sequences at different positions in one T-query call (B*T*Hkv =
    640 slots, so the bf16 scoring is bucketed by parent across filing blocks
    of both sequences): sampled queries equal the single-query (per-query
    scoring) path exactly, and the oracle."""
    _need_gpu()
    B, Hkv, d, k, T = 2, 2, 128, 16, 160
    L0 = 8192 + 37
    L_cap = L0 + T + 16
    wl, tree, pool, pdict = _setup(B, Hkv, d, L_cap, L_cap, k, "bf16", 41)
    assert tree.n_levels == 4
    R.recsa_build_tree(tree, pool, 0, L0 + T)
    Hq = Hkv * 4
    q = synth.to_storage(synth.normal((B, T, Hq, d), DEV, 41, 97), "bf16")
    pos = (torch.arange(L0, L0 + T, device=DEV).view(1, T)
           - 5 * torch.arange(B, device=DEV).view(B, 1)).contiguous()
    sel, cnt, imp, out = _run_select_attn(tree, q, Hq, pos, decode=False)
    idx = [0, 77, T - 1]
    for i in idx:
        s2, c2, m2, o2 = _run_select_attn(tree, q[:, i:i + 1].contiguous(), Hq,
                                          pos[:, i:i + 1].contiguous(), decode=True)
        assert np.array_equal(s2[:, 0], sel[:, i]) and np.array_equal(c2[:, 0], cnt[:, i])
        assert np.array_equal(m2[:, 0], imp[:, i])
    rep = _check_queries(tree, pdict, q[:, idx], pos[:, idx].cpu(), sel[:, idx], cnt[:, idx],
                         imp[:, idx], out[:, idx], [0, 1], 2e-3)
    assert rep.compared == B * 2 * len(idx) and rep.imp_levels > 0, rep


def test_k512_variant_decode_and_prefill():
    """The pages' k = 512 ablation (C*k = 8192 list positions, a top-(k-1)
    over up to 8191 keys): 120K tokens give 3 levels whose level-1 lists hold
    about 7500 candidates.  A causal prefill chunk (bucketed scoring), then
    the fused decode against the separate calls, sampled vs the oracle."""
    _need_gpu()
    L0, T, Hkv, Hq = 120000, 256, 2, 8
    L_cap = L0 + T + 64
    wl, tree, pool, pdict = _setup(1, Hkv, 128, L_cap, L_cap, 512, "bf16", 51)
    assert tree.n_levels == 3
    R.recsa_build_tree(tree, pool, 0, L0)
    R.recsa_build_tree(tree, pool, L0, L0 + T)
    q = synth.to_storage(synth.normal((1, T, Hq, 128), DEV, 51, 97), "bf16")
    pos = torch.arange(L0, L0 + T, device=DEV).view(1, T)
    sel, cnt, imp, out = _run_select_attn(tree, q, Hq, pos, decode=False)
    idx = [0, 100, T - 1]
    rep = _check_queries(tree, pdict, q[:, idx], pos[:, idx].cpu(), sel[:, idx], cnt[:, idx],
                         imp[:, idx], out[:, idx], [0, 1], 2e-3)
    assert rep.compared == 2 * len(idx) and rep.imp_levels > 0, rep
    t = L0 + T
    kn, vn = tree.K[0][:, :, t].clone().contiguous(), tree.V[0][:, :, t].clone().contiguous()
    qd = synth.to_storage(synth.normal((1, 1, Hq, 128), DEV, 51, 98), "bf16")
    p1 = torch.tensor([t], dtype=torch.int64, device=DEV)
    ref = R.Tree.allocate(1, Hkv, 128, L_cap, k=512, dtype="bf16", device=DEV,
                          level0=(tree.K[0].clone(), tree.V[0].clone()))
    R.recsa_build_tree(ref, pool, 0, L0 + T)
    fs, fc, fo, ws = _fused_step(tree, pool, kn, vn, qd, Hq, p1)
    R.recsa_append_decode(ref, pool, kn, vn, p1)
    s2, c2, m2, o2 = _run_select_attn(ref, qd, Hq, p1.view(1, 1), decode=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(R.decode_error_words(ws, tree, Hq)).item() == 0
    assert np.array_equal(fs.cpu().numpy().reshape(s2.shape), s2)
    assert np.allclose(fo.cpu().numpy().astype(np.float64).reshape(o2.shape), o2, rtol=0,
                       atol=1e-5 * np.abs(o2).max())
    rep2 = _check_queries(ref, pdict, qd, p1.view(1, 1).cpu(), s2, c2, m2, o2, [0, 1], 2e-3)
    assert rep2.compared == 2 and rep2.imp_levels > 0, rep2


def test_fused_decode_variable_lengths():
    """Sequences of very different lengths in one decode batch: t = 70000 (two
    scored levels), 5000 (one) and 300 (none: every list fits in k), so the
    groups of one launch run different numbers of selection handoffs.  The
    fused step equals the separate calls, and each sequence the oracle."""
    _need_gpu()
    B, Hkv, d, k = 3, 2, 128, 256
    L_cap = 70100
    ts = [70000, 5000, 300]
    wl, tree, pool, pdict = _setup(B, Hkv, d, L_cap, L_cap, k, "bf16", 61)
    assert tree.n_levels == 4
    ref = R.Tree.allocate(B, Hkv, d, L_cap, k=k, dtype="bf16", device=DEV,
                          level0=(tree.K[0].clone(), tree.V[0].clone()))
    R.recsa_build_tree(tree, pool, 0, max(ts))
    R.recsa_build_tree(ref, pool, 0, max(ts))
    Hq = Hkv * 4
    pos = torch.tensor(ts, dtype=torch.int64, device=DEV)
    kn = torch.stack([tree.K[0][b, :, ts[b]] for b in range(B)]).contiguous()
    vn = torch.stack([tree.V[0][b, :, ts[b]] for b in range(B)]).contiguous()
    q = synth.to_storage(synth.normal((B, 1, Hq, d), DEV, 61, 99), "bf16")
    fs, fc, fo, ws = _fused_step(tree, pool, kn, vn, q, Hq, pos)
    R.recsa_append_decode(ref, pool, kn, vn, pos)
    s2, c2, m2, o2 = _run_select_attn(ref, q, Hq, pos.view(B, 1), decode=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(R.decode_error_words(ws, tree, Hq)).item() == 0
    assert torch.count_nonzero(R.decode_control_words(ws, tree, Hq)).item() == 0
    assert np.array_equal(fs.cpu().numpy().reshape(s2.shape), s2)
    assert np.array_equal(fc.cpu().numpy().reshape(c2.shape), c2)
    assert np.allclose(fo.cpu().numpy().astype(np.float64).reshape(o2.shape), o2, rtol=0,
                       atol=1e-5 * np.abs(o2).max())
    compared = 0
    for b in range(B):
        rep = _check_queries(ref, pdict, q[b:b + 1], pos[b:b + 1].view(1, 1).cpu(), s2[b:b + 1],
                             c2[b:b + 1], m2[b:b + 1], o2[b:b + 1], [0, 1], 2e-3, seqs=[b])
        compared += rep.compared
    assert compared == 2 * B


@pytest.mark.skip(reason="G = 8 query heads per KV head is switched off (RECSA_E_UNSUPPORTED): "
                         "its one fused-decode GPU run (B = 3, Hkv = 2) failed, and the cause "
                         "of that failure has not been shown.  Its 256-VGPR / 76-byte-spill / "
                         "119 KB-LDS build and the since-fixed scoring store of MFMA rows 4-7 "
                         "are recorded; it is not run on the GPU until a cause is shown.")
def test_fused_decode_g8_matches_separate_calls():
    """The fused decode at G = 8 (B = 3, Hkv = 2, bf16 d = 128) against the
    separate calls and the oracle -- the case that failed once."""
    _need_gpu()
    test_fused_decode_matches_separate_calls("bf16", 128, 2, 8, 3)
