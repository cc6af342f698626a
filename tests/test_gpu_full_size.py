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

from tests.test_gpu_parity import _check_queries, _need_gpu

pytestmark = pytest.mark.gpu


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
    n_sel, k = tree.n_sel, tree.k
    trees = {}

    # decode: KV heads 0 and 5, all four query heads of each
    sel = w.sel_dec.cpu().numpy().reshape(B, 1, tree.Hkv, n_sel, k)
    cnt = w.cnt_dec.cpu().numpy().reshape(B, 1, tree.Hkv, n_sel)
    out = w.out_dec.cpu().numpy().astype(np.float64).reshape(B, 1, Hq, tree.d)
    pos = w.pos_dec.view(B, 1).cpu()
    print(f"decode at t={int(pos[0, 0])}: checking KV heads 0, 5", flush=True)
    rep = _check_queries(tree, w.pdict, w.q_dec, pos, sel, cnt, None, out, [0, 5],
                         1e-5, 2e-3, trees={}, max_swaps=1)
    assert rep.matched >= 1, rep

    # prefill chunk: 4 queries spread over the chunk, KV head 2
    idx = [0, 1, T // 2, T - 1]
    sel_p = w.sel_pre.cpu().numpy().reshape(B, T, tree.Hkv, n_sel, k)[:, idx]
    cnt_p = w.cnt_pre.cpu().numpy().reshape(B, T, tree.Hkv, n_sel)[:, idx]
    out_p = w.out_pre.cpu().numpy().astype(np.float64)[:, idx]
    pos_p = w.pos_pre[:, idx].cpu()
    print(f"prefill chunk: checking queries at {pos_p[0].tolist()} on KV head 2", flush=True)
    rep2 = _check_queries(tree, w.pdict, w.q_pre[:, idx], pos_p, sel_p, cnt_p, None, out_p,
                          [2], 1e-5, 2e-3, trees=trees, max_swaps=1)
    assert rep2.matched >= len(idx) - 1, rep2
