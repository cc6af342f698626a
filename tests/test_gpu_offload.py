"""Level 0 of the KV cache in host memory (picx.dev Efficiency Results: KV
offloading at 1M/2M tokens; Practical Implications: only the levels above
level 0 and the gathered exact tokens occupy GPU memory).

K[0], V[0] and Kr[0] live in pinned host memory and the kernels read the
selected 16-row groups of level 0 over PCIe in place; levels >= 1 stay in
HBM.  Bar: every call gives bit-identical results to the same tree with level
0 in device memory (whose parity with the oracle the other GPU tests
establish), and sampled queries match the oracle directly.
"""

import numpy as np
import pytest
import torch

import synth
from tests import test_gpu_parity as TP

pytestmark = pytest.mark.gpu

R = pytest.importorskip("long_context_kv_amd.recsa")
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R.lib()


def _pair(B, Hkv, d, L_cap, k, dtype, seed):
    """The same level-0 rows in a device-resident tree and a host-resident
    one, plus the pooler."""
    wl = synth.Workload("offload", B, Hkv, Hkv * 4, d, dtype, L_cap, 16, k, seed)
    K, V = synth.kv_rows(wl, DEV, n_rows=L_cap)
    pdict = synth.pooler_params(d, d, DEV, seed)
    dev = R.Tree.allocate(B, Hkv, d, L_cap, k=k, dtype=dtype, device=DEV, level0=(K, V))
    host = R.Tree.allocate(B, Hkv, d, L_cap, k=k, dtype=dtype, device=DEV, level0=(K, V),
                           level0_host=True)
    assert host.K[0].device.type == "cpu" and host.K[0].is_pinned()
    assert host.level0_dptr is not None and all(host.level0_dptr[:2])
    assert (host.level0_dptr[2] is None) == (host.Kr[0].numel() == 0)
    return dev, host, R.Pooler.from_dict(pdict, DEV), pdict


def _same_tree(a, b):
    for lvl in range(a.n_levels):
        for name in ("K", "V", "Kr"):
            x, y = getattr(a, name)[lvl], getattr(b, name)[lvl]
            assert torch.equal(x.cpu(), y.cpu()), (name, lvl)


def test_offloaded_level0_matches_device_resident():
    """40K tokens, two sequences, k = 64 (two scored levels): build, a causal
    prefill chunk, the fused decode and the separate decode calls, with level
    0 in host memory, against the device-resident tree bit for bit; sampled
    prefill queries against the oracle."""
    _need_gpu()
    L0, T, B, Hkv, d, k = 40000, 128, 2, 2, 128, 64
    L_cap = L0 + T + 64
    dev, host, pool, pdict = _pair(B, Hkv, d, L_cap, k, "bf16", 71)
    for tr in (dev, host):
        R.recsa_build_tree(tr, pool, 0, L0)
        R.recsa_build_tree(tr, pool, L0, L0 + T)
    torch.cuda.synchronize()
    _same_tree(dev, host)

    Hq = Hkv * 4
    q = synth.to_storage(synth.normal((B, T, Hq, d), DEV, 71, 5), "bf16")
    pos = torch.arange(L0, L0 + T, device=DEV).view(1, T).repeat(B, 1).contiguous()
    pos[1] -= 7
    r_dev = TP._run_select_attn(dev, q, Hq, pos, decode=False)
    r_host = TP._run_select_attn(host, q, Hq, pos, decode=False)
    for a, b in zip(r_dev, r_host):
        assert np.array_equal(a, b)
    sel, cnt, imp, out = r_host
    idx = [0, T - 1]
    rep = TP._check_queries(host, pdict, q[:, idx], pos[:, idx].cpu(), sel[:, idx],
                            cnt[:, idx], imp[:, idx], out[:, idx], [0, 1], 2e-3)
    assert rep.compared == 2 * len(idx) * 2 and rep.imp_levels > 0, rep

    # one decode step at t = L0 + T (fused), then the same step as three calls
    t = L0 + T
    kn = synth.to_storage(synth.normal((B, Hkv, d), DEV, 71, 6), "bf16")
    vn = synth.to_storage(synth.normal((B, Hkv, d), DEV, 71, 7), "bf16")
    qd = synth.to_storage(synth.normal((B, 1, Hq, d), DEV, 71, 8), "bf16")
    p1 = torch.full((B,), t, dtype=torch.int64, device=DEV)
    res = []
    for tr in (dev, host):
        fs, fc, fo, ws = TP._fused_step(tr, pool, kn, vn, qd, Hq, p1)
        torch.cuda.synchronize()
        assert torch.count_nonzero(R.decode_error_words(ws, tr, Hq)).item() == 0
        res.append((fs.cpu(), fc.cpu(), fo.cpu()))
    for a, b in zip(*res):
        assert torch.equal(a, b)
    _same_tree(dev, host)                     # the appended row and completed nodes
    assert torch.equal(host.K[0][:, :, t], kn.cpu())
    # separate calls on the host-resident tree (the row is appended again: same bits)
    R.recsa_append_decode(host, pool, kn, vn, p1)
    s2, c2, m2, o2 = TP._run_select_attn(host, qd, Hq, p1.view(B, 1), decode=True)
    assert np.array_equal(s2.reshape(-1), res[1][0].numpy().reshape(-1))
    assert np.allclose(o2.reshape(-1), res[1][2].numpy().astype(np.float64).reshape(-1),
                       rtol=0, atol=1e-5 * np.abs(o2).max())


def test_offloaded_level0_fp32_small():
    """The tiny shape (fp32, d = 64, one KV head, k = 16) with level 0 in
    host memory: every position class of a 4096-token tree, against the
    device-resident tree bit for bit."""
    _need_gpu()
    L0, d, k = 4096, 64, 16
    dev, host, pool, pdict = _pair(1, 1, d, L0, k, "f32", 72)
    for tr in (dev, host):
        R.recsa_build_tree(tr, pool, 0, L0)
    torch.cuda.synchronize()
    _same_tree(dev, host)
    ts = [0, 1, 15, 16, 255, 256, 1000, 4095]
    T = len(ts)
    q = synth.normal((1, T, 4, d), DEV, 72, 5)
    pos = torch.tensor([ts], dtype=torch.int64, device=DEV)
    r_dev = TP._run_select_attn(dev, q, 4, pos, decode=False)
    r_host = TP._run_select_attn(host, q, 4, pos, decode=False)
    for a, b in zip(r_dev, r_host):
        assert np.array_equal(a, b)


def test_offloaded_level0_524k_bench_shape_matches_device_resident():
    """The 524K workload shape as `bench.py --offload` runs it (8 KV heads,
    32 query heads, d = 128, k = 256, 4 levels): full build, a 256-query
    causal chunk and the fused decode after it, with level 0 in host memory,
    bit for bit against the same steps on the device-resident tree."""
    _need_gpu()
    wl = synth.WORKLOADS["524k"]
    L, T = wl.L, 256
    t_dec = L + T
    L_cap = t_dec + 64
    K, V = synth.kv_rows_device(wl, DEV, L_cap)
    pdict = synth.pooler_params(wl.d, wl.d, DEV, wl.seed)
    pool = R.Pooler.from_dict(pdict, DEV)
    dev = R.Tree.allocate(1, wl.Hkv, wl.d, L_cap, k=wl.k, dtype="bf16", device=DEV, level0=(K, V))
    host = R.Tree.allocate(1, wl.Hkv, wl.d, L_cap, k=wl.k, dtype="bf16", device=DEV,
                           level0=(K, V), level0_host=True)
    q_pre = synth.to_storage(synth.normal((1, T, wl.Hq, wl.d), DEV, wl.seed, 41), "bf16")
    q_dec = synth.decode_queries(wl, DEV)
    kn = K[:, :, t_dec].clone().contiguous()
    vn = V[:, :, t_dec].clone().contiguous()
    pos = torch.arange(L, L + T, device=DEV).view(1, T)
    p1 = torch.tensor([t_dec], dtype=torch.int64, device=DEV)
    res = []
    for tr in (dev, host):
        print("524K offload:", "host" if tr is host else "device", flush=True)
        R.recsa_build_tree(tr, pool, 0, L)
        R.recsa_build_tree(tr, pool, L, L + T)
        r = TP._run_select_attn(tr, q_pre, wl.Hq, pos, decode=False)
        fs, fc, fo, ws = TP._fused_step(tr, pool, kn, vn, q_dec, wl.Hq, p1)
        torch.cuda.synchronize()
        assert torch.count_nonzero(R.decode_error_words(ws, tr, wl.Hq)).item() == 0
        res.append(list(r) + [fs.cpu().numpy(), fo.cpu().numpy()])
        del ws
    for a, b in zip(*res):
        assert np.array_equal(a, b)
    for lvl in range(1, dev.n_levels):
        assert torch.equal(dev.K[lvl], host.K[lvl]) and torch.equal(dev.Kr[lvl], host.Kr[lvl])
    assert torch.equal(dev.Kr[0].cpu(), host.Kr[0])
