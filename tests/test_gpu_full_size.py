"""Full-size parity: the 524K-token model-shaped workload (8 KV heads, 32 query
heads, d=128, bf16, C=16, k=256) in exactly the launch configuration the
benchmark times -- full tree build, a causal 4096-query prefill chunk
(incremental build, T-query selection and attention) and the single-launch
decode step at t = 528384 -- with sampled outputs checked one by one against
the CPU oracle (sampled KV heads for the decode, sampled chunk queries for the
prefill), to the same bars as the small parity tests."""

import numpy as np
import pytest
import torch

import synth
from long_context_kv_amd import recsa as R
from tests.test_gpu_parity import DEV, _check_queries, _need_gpu

pytestmark = pytest.mark.gpu


def _select_with_importance(tree, q, Hq, T, pos, sel_ref, cnt_ref):
    """Run the selection again with importances (same launch shape and
    workspace size as the timed call) and require the same bits for the
    selection; returns the selection, counts and importances as arrays
    [B][T][Hkv][...]."""
    B = pos.shape[0]
    ws = R.workspace(tree, Hq, B * T)
    sel, cnt, imp = tree.selection_buffers(B * T, with_importance=True)
    R.recsa_select(tree, q, Hq, T, pos.reshape(B, T), sel, cnt, imp, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel.view(-1), sel_ref.view(-1)) and torch.equal(cnt.view(-1), cnt_ref.view(-1))
    shp = (B, T, tree.Hkv, tree.n_sel)
    out = (sel.cpu().numpy().reshape(*shp, tree.k), cnt.cpu().numpy().reshape(shp),
           imp.cpu().numpy().reshape(*shp, -1))
    del ws, imp
    return out


def test_524k_bench_configuration_sampled_vs_oracle():
    _need_gpu()
    import bench
    w = bench.setup_workload("524k")
    tree, B, T, Hq = w.tree, w.wl.B, w.T, w.wl.Hq
    w.build_full()
    w.prefill()
    w.decode()
    torch.cuda.synchronize()
    err = w.R.decode_error_words(w.ws_dec, tree, Hq)
    assert torch.count_nonzero(err).item() == 0
    trees = {}

    # decode: KV heads 0 and 5, all four query heads of each; the fused
    # step's selection equals the separate selection call's, whose
    # importances are compared too
    sel, cnt, imp = _select_with_importance(tree, w.q_dec, Hq, 1, w.pos_dec, w.sel_dec, w.cnt_dec)
    out = w.out_dec.cpu().numpy().astype(np.float64).reshape(B, 1, Hq, tree.d)
    pos = w.pos_dec.view(B, 1).cpu()
    print(f"decode at t={int(pos[0, 0])}: checking KV heads 0, 5", flush=True)
    rep = _check_queries(tree, w.pdict, w.q_dec, pos, sel, cnt, imp, out, [0, 5],
                         2e-3, trees=trees)
    assert rep.compared == 2 and rep.imp_levels == 2 * 2, rep

    # prefill chunk: 4 queries spread over the chunk, KV head 2
    idx = [0, 1, T // 2, T - 1]
    sel_p, cnt_p, imp_p = _select_with_importance(tree, w.q_pre, Hq, T, w.pos_pre, w.sel_pre,
                                                  w.cnt_pre)
    out_p = w.out_pre.cpu().numpy().astype(np.float64)[:, idx]
    pos_p = w.pos_pre[:, idx].cpu()
    print(f"prefill chunk: checking queries at {pos_p[0].tolist()} on KV head 2", flush=True)
    rep2 = _check_queries(tree, w.pdict, w.q_pre[:, idx], pos_p, sel_p[:, idx], cnt_p[:, idx],
                          imp_p[:, idx], out_p, [2], 2e-3, trees=trees)
    assert rep2.compared == len(idx) and rep2.imp_levels == 2 * len(idx), rep2


def test_1m_batch4_decode_sampled_vs_oracle():
    """1M tokens, 4 independent sequences (5 tree levels, 3 of them scored),
    each at its own position, through the single-launch decode in the
    benchmark's launch configuration; sampled (sequence, KV head) pairs vs
    the oracle.  Nodes past a sequence's own position are built too (its walk
    never reads a node past its current node)."""
    _need_gpu()
    wl = synth.WORKLOADS["1m_b4"]
    L, B = wl.L, wl.B
    L_cap = L + 64
    K, V = synth.kv_rows_device(wl, DEV, L_cap)
    q = synth.decode_queries(wl, DEV)                          # [B, 1, Hq, d]
    synth.plant_needles(wl, K[:, :, :L], q)
    pdict = synth.pooler_params(wl.d, wl.d, DEV, wl.seed)
    pool = R.Pooler.from_dict(pdict, DEV)
    tree = R.Tree.allocate(B, wl.Hkv, wl.d, L_cap, k=wl.k, dtype="bf16", device=DEV,
                           level0=(K, V))
    assert tree.n_levels == 5
    t_b = [L - 3 * b for b in range(B)]
    R.recsa_build_tree(tree, pool, 0, L)
    pos = torch.tensor(t_b, dtype=torch.int64, device=DEV)
    kn = torch.stack([K[b, :, t_b[b]] for b in range(B)]).contiguous()
    vn = torch.stack([V[b, :, t_b[b]] for b in range(B)]).contiguous()
    ws = R.workspace(tree, wl.Hq, B)
    sel, cnt, _ = tree.selection_buffers(B)
    out = torch.empty((B, wl.Hq, wl.d), dtype=torch.float32, device=DEV)
    R.recsa_decode(tree, pool, kn, vn, q, wl.Hq, pos, sel, cnt, out, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(R.decode_error_words(ws, tree, wl.Hq)).item() == 0
    del ws
    s_np, c_np, i_np = _select_with_importance(tree, q, wl.Hq, 1, pos, sel, cnt)
    o_np = out.cpu().numpy().astype(np.float64).reshape(B, 1, wl.Hq, wl.d)
    compared = 0
    for b, j in ((0, 0), (1, 3), (3, 7)):
        print(f"1M x 4 decode: sequence {b} at t={t_b[b]}, KV head {j}", flush=True)
        rep = _check_queries(tree, pdict, q[b:b + 1], pos[b:b + 1].view(1, 1).cpu(),
                             s_np[b:b + 1], c_np[b:b + 1], i_np[b:b + 1], o_np[b:b + 1], [j],
                             2e-3, trees={}, seqs=[b])
        assert rep.imp_levels >= 2, rep          # sequence 3 at t < 2^20 scores two levels
        compared += rep.compared
    assert compared == 3


def test_2m_layer_decode_and_prefill_sampled_vs_oracle():
    """One layer of the 2M-token workload: full build over 2M tokens, an
    8192-query causal prefill chunk (incremental build, T-query selection and
    attention) and the single-launch decode right after it; sampled queries
    and KV heads vs the oracle."""
    _need_gpu()
    wl = synth.WORKLOADS["2m_l4"]
    L, T = wl.L, wl.prefill_T
    t_dec = L + T
    L_cap = t_dec + 64
    K, V = synth.kv_rows_device(wl, DEV, L_cap)
    q_dec = synth.decode_queries(wl, DEV)
    synth.plant_needles(wl, K[:, :, :L], q_dec)
    q_pre = synth.new_rows(wl, DEV, T, "chunk")[2]             # [1, T, Hq, d]
    pdict = synth.pooler_params(wl.d, wl.d, DEV, wl.seed)
    pool = R.Pooler.from_dict(pdict, DEV)
    tree = R.Tree.allocate(1, wl.Hkv, wl.d, L_cap, k=wl.k, dtype="bf16", device=DEV,
                           level0=(K, V))
    R.recsa_build_tree(tree, pool, 0, L)
    R.recsa_build_tree(tree, pool, L, L + T)
    pos_pre = torch.arange(L, L + T, device=DEV).view(1, T)
    ws = R.workspace(tree, wl.Hq, T)
    sel, cnt, _ = tree.selection_buffers(T)
    R.recsa_select(tree, q_pre, wl.Hq, T, pos_pre, sel, cnt, None, ws)
    out_pre = torch.empty((1, T, wl.Hq, wl.d), dtype=torch.float32, device=DEV)
    R.recsa_attn_prefill(tree, q_pre, wl.Hq, T, pos_pre, sel, cnt, out_pre, ws)
    del ws
    pos = torch.tensor([t_dec], dtype=torch.int64, device=DEV)
    wsd = R.workspace(tree, wl.Hq, 1)
    seld, cntd, _ = tree.selection_buffers(1)
    outd = torch.empty((1, wl.Hq, wl.d), dtype=torch.float32, device=DEV)
    R.recsa_decode(tree, pool, K[:, :, t_dec].contiguous(), V[:, :, t_dec].contiguous(), q_dec,
                   wl.Hq, pos, seld, cntd, outd, wsd)
    torch.cuda.synchronize()
    assert torch.count_nonzero(R.decode_error_words(wsd, tree, wl.Hq)).item() == 0
    del wsd
    trees = {}
    print(f"2M decode at t={t_dec}: KV heads 1, 6", flush=True)
    sd, cd, idd = _select_with_importance(tree, q_dec, wl.Hq, 1, pos, seld, cntd)
    rep = _check_queries(tree, pdict, q_dec, pos.view(1, 1).cpu(), sd, cd, idd,
                         outd.cpu().numpy().astype(np.float64).reshape(1, 1, wl.Hq, wl.d),
                         [1, 6], 2e-3, trees=trees)
    assert rep.compared == 2 and rep.imp_levels == 2 * 3, rep
    idx = [0, T // 3, T - 1]
    print(f"2M prefill chunk: queries {[L + i for i in idx]} on KV head 6", flush=True)
    sp, cp, ip = _select_with_importance(tree, q_pre, wl.Hq, T, pos_pre, sel, cnt)
    rep2 = _check_queries(tree, pdict, q_pre[:, idx], pos_pre[:, idx].cpu(), sp[:, idx],
                          cp[:, idx], ip[:, idx],
                          out_pre.cpu().numpy().astype(np.float64)[:, idx], [6],
                          2e-3, trees=trees)
    assert rep2.compared == len(idx) and rep2.imp_levels == 3 * len(idx), rep2


def test_config5_4layers_2m_last_decode_step_sampled_vs_oracle():
    """The 4-layer 2M-token configuration exactly as the benchmark runs it
    (class Config5): all four layers resident, the full build and the
    8192-query chunk of every layer, then 256 decode steps of the four layers
    with fresh inputs.  The last step (token L + 8192 + 255) of the last
    layer is checked on two KV heads against the oracle; its selection is
    run again with importances (same bits), which are compared too."""
    _need_gpu()
    import bench
    torch.cuda.empty_cache()
    c = bench.Config5()
    for ly in range(c.n_layers):
        c.build(ly)
    for ly in range(c.n_layers):
        c.prefill(ly)
    for s_ in range(c.steps):
        c.decode(s_)
    torch.cuda.synchronize()
    ly = c.n_layers - 1
    x = c.layers[ly]
    tree, Hq = x["tree"], c.wl.Hq
    assert torch.count_nonzero(R.decode_error_words(c.ws_dec, tree, Hq)).item() == 0
    q, _, _, pos = x["dec"][c.steps - 1]
    sel_d, cnt_d = c.sel_dec[ly]
    out = c.out_dec[ly].cpu().numpy().astype(np.float64).reshape(1, 1, Hq, tree.d)
    del c.ws_pre
    torch.cuda.empty_cache()
    sd, cd, idd = _select_with_importance(tree, q, Hq, 1, pos, sel_d, cnt_d)
    print(f"config 5: layer {ly}, decode step {c.steps - 1} at t={int(pos[0])}: KV heads 2, 7",
          flush=True)
    rep = _check_queries(tree, x["pdict"], q, pos.view(1, 1).cpu(), sd, cd, idd, out, [2, 7],
                         2e-3)
    assert rep.compared == 2 and rep.imp_levels == 2 * 3, rep


def test_distill_32k_bench_configuration_sampled_vs_oracle():
    """The distillation workload exactly as `bench.py --distill` runs it: a
    32768-token tree at k = 64, every position a query (selection with
    importances, Eq. 6 terms), the Eq. 7 penalty over every node, and the
    pooler backward of levels 1 and 2 with the benchmark's seeded key
    gradients, the KL key gradient of every position; sampled queries and
    heads against the oracle, the penalty and the pooler gradients over all
    heads, to the small tests' bars."""
    _need_gpu()
    import bench
    from oracle import recsa_oracle as O
    from tests import parity as PY
    from tests import test_gpu_distill as TD
    from tests import test_gpu_pool_backward as TB
    wl = synth.WORKLOADS["distill_32k"]
    L, B, Hkv, Hq, d = wl.L, wl.B, wl.Hkv, wl.Hq, wl.d
    K0, V0 = synth.kv_rows(wl, DEV, n_rows=L)
    pdict = synth.pooler_params(d, d, DEV, wl.seed)
    pool = R.Pooler.from_dict(pdict, DEV)
    tree = R.Tree.allocate(B, Hkv, d, L, k=wl.k, dtype=wl.dtype, device=DEV, level0=(K0, V0),
                           theta=wl.theta)
    R.recsa_build_tree(tree, pool, 0, L)
    q = synth.to_storage(synth.normal((B, L, Hq, d), DEV, wl.seed, bench.ROLE_DISTILL_Q),
                         wl.dtype)
    pos = torch.arange(L, device=DEV).view(1, L).contiguous()
    sel, cnt, imp, kl = TD.run_distill(tree, q, Hq, pos)
    assert np.all(np.isfinite(kl)) and np.all(kl >= -1e-6)
    idx = [1023, 1024, 16383, L - 1]
    print(f"distill 32K: queries {idx} on KV heads 0, 5", flush=True)
    for j in (0, 5):
        n_pairs, n_lv, worst = TD.check_kl(tree, pdict, q[:, idx], pos[:, idx].cpu(), sel[:, idx],
                                           cnt[:, idx], imp[:, idx], kl[:, idx], [j])
        assert n_pairs == len(idx) and n_lv >= 2, (j, n_pairs, n_lv)
    # Eq. 7 over every node of every head, and the backward of levels 1, 2
    print("distill 32K: shift penalty and pooler backward, all heads", flush=True)
    sws = torch.empty(R.recsa_shift_workspace_bytes(tree), dtype=torch.uint8, device=DEV)
    pen = torch.zeros((tree.n_levels - 1, d + 2), dtype=torch.float32, device=DEV)
    R.recsa_shift_penalty(tree, pool, L, pen, sws)
    torch.cuda.synchronize()
    g = pen.cpu().numpy().astype(np.float64)
    ref = TD._shift_oracle(tree, pdict, L)
    for lvl, (s, mu2, p) in ref.items():
        assert np.max(np.abs(g[lvl - 1, :d] - s)) <= 1e-4 * np.max(np.abs(s)), lvl
        assert abs(g[lvl - 1, d] - mu2) <= 1e-5 * mu2, lvl
        assert abs(g[lvl - 1, d + 1] - p) <= 1e-4 * p, lvl
    for lv in (2, 1):
        dK = synth.normal((B, Hkv, R.recsa_level_rows(L, 16, lv), d), DEV, wl.seed, 20 + lv)
        gg = TB.gpu_backward(tree, pool, lv, L, dK, 1.0)
        TB.compare(gg, TB.oracle_backward(tree, pdict, lv, L, dK, 1.0),
                   1e-3 if lv > 1 else 1e-4)
    # KL key gradient: every position in one launch, as the benchmark runs it
    # (finite, identical bits on a second call, nothing at the top level,
    # whose list never exceeds k); the sampled queries alone against the
    # oracle (the gradient is a sum over queries)
    from tests import test_gpu_kl_backward as TK
    print("distill 32K: KL key gradient, every position", flush=True)
    _, _, _, full = TK.run_key_grad(tree, q, Hq, pos)
    for l, v in enumerate(full):
        assert np.all(np.isfinite(v)), l + 1
    assert np.all(full[-1] == 0.0) and np.any(full[0] != 0.0)
    print(f"distill 32K: KL key gradient of queries {idx} one at a time vs oracle, KV heads 0, 5",
          flush=True)
    n_cmp, n_scored = 0, 0
    for i in idx:
        qs, ps = q[:, [i]].contiguous(), pos[:, [i]].contiguous()
        sel_s, cnt_s, imp_s, dKs = TK.run_key_grad(tree, qs, Hq, ps)
        c, sc = TK.compare_with_oracle(tree, pdict, qs, ps.cpu(), sel_s, cnt_s, imp_s, dKs, (0, 5),
                                       TK.tolerance(2e-4, 16 * wl.k))
        n_cmp += c
        n_scored += int(sc)
    assert n_cmp == 2 * len(idx) and n_scored >= len(idx) - 2, (n_cmp, n_scored)
