"""Trees without the rotated-key copy Kr (every Kr[l] NULL: the C ABI's K/V-
only contract, levels >= 1 adding 1/15 of the cache): the kernels rotate the
key rows they read by their in-group offset, with the float32 rotation and
rounding the stored copy holds, so every call gives the same bits as on the
same tree with Kr -- checked for the build, a prefill chunk (bucketed bf16
scoring and float32 per-query scoring), the fused decode, the separate decode
calls and level 0 in host memory; sampled queries against the oracle."""

import numpy as np
import pytest
import torch

import synth
from tests import test_gpu_parity as TP

pytestmark = pytest.mark.gpu

R = pytest.importorskip("long_context_kv_amd.recsa")
DEV = "cuda"


def _pair(B, Hkv, d, L_cap, k, dtype, seed, level0_host=False):
    wl = synth.Workload("nokr", B, Hkv, Hkv * 4, d, dtype, L_cap, 16, k, seed)
    K, V = synth.kv_rows(wl, DEV, n_rows=L_cap)
    pdict = synth.pooler_params(d, d, DEV, seed)
    with_kr = R.Tree.allocate(B, Hkv, d, L_cap, k=k, dtype=dtype, device=DEV,
                              level0=(K.clone(), V.clone()))
    no_kr = R.Tree.allocate(B, Hkv, d, L_cap, k=k, dtype=dtype, device=DEV,
                            level0=(K.clone(), V.clone()), rotated_keys=False,
                            level0_host=level0_host)
    assert all(x.numel() == 0 for x in no_kr.Kr)
    return with_kr, no_kr, R.Pooler.from_dict(pdict, DEV), pdict


@pytest.mark.parametrize("dtype,d,k,L0,T,B,Hkv,host", [
    ("bf16", 128, 64, 40000, 128, 2, 2, False),     # bucketed scoring (512 slots)
    ("f32", 64, 16, 5000, 40, 1, 2, False),         # per-query float32 scoring
    ("bf16", 128, 64, 40000, 64, 1, 2, True),       # level 0 in host memory
])
def test_without_rotated_keys_equals_with(dtype, d, k, L0, T, B, Hkv, host):
    TP._need_gpu()
    L_cap = L0 + T + 64
    a, b, pool, pdict = _pair(B, Hkv, d, L_cap, k, dtype, 81, host)
    for tr in (a, b):
        R.recsa_build_tree(tr, pool, 0, L0)
        R.recsa_build_tree(tr, pool, L0, L0 + T)
    torch.cuda.synchronize()
    for lvl in range(a.n_levels):
        assert torch.equal(a.K[lvl].cpu(), b.K[lvl].cpu()) and \
            torch.equal(a.V[lvl].cpu(), b.V[lvl].cpu()), lvl
    Hq = Hkv * 4
    q = synth.to_storage(synth.normal((B, T, Hq, d), DEV, 81, 1), dtype)
    pos = (torch.arange(L0, L0 + T, device=DEV).view(1, T)
           - 3 * torch.arange(B, device=DEV).view(B, 1)).contiguous()
    ra = TP._run_select_attn(a, q, Hq, pos, decode=False)
    rb = TP._run_select_attn(b, q, Hq, pos, decode=False)
    for x, y in zip(ra, rb):
        assert np.array_equal(x, y)
    # one decode step: fused on the tree without Kr, separate calls, and the
    # fused step on the tree with Kr
    t = L0 + T
    kn = synth.to_storage(synth.normal((B, Hkv, d), DEV, 81, 2), dtype)
    vn = synth.to_storage(synth.normal((B, Hkv, d), DEV, 81, 3), dtype)
    qd = synth.to_storage(synth.normal((B, 1, Hq, d), DEV, 81, 4), dtype)
    p1 = torch.full((B,), t, dtype=torch.int64, device=DEV)
    fa = TP._fused_step(a, pool, kn, vn, qd, Hq, p1)
    fb = TP._fused_step(b, pool, kn, vn, qd, Hq, p1)
    torch.cuda.synchronize()
    for x, y in zip(fa[:3], fb[:3]):
        assert torch.equal(x, y)
    assert torch.count_nonzero(R.decode_control_words(fb[3], b, Hq)).item() == 0
    R.recsa_append_decode(b, pool, kn, vn, p1)
    s2, c2, m2, o2 = TP._run_select_attn(b, qd, Hq, p1.view(B, 1), decode=True)
    assert np.array_equal(s2.reshape(-1), fb[0].cpu().numpy().reshape(-1))
    sa, ca, ma, oa = TP._run_select_attn(a, qd, Hq, p1.view(B, 1), decode=True)
    assert np.array_equal(o2, oa) and np.array_equal(m2, ma)
    # the tree without Kr against the oracle (staged protocol)
    idx = [0, T - 1]
    tol = 1e-5 if dtype == "f32" else 2e-3
    sel, cnt, imp, out = rb
    rep = TP._check_queries(b, pdict, q[:, idx], pos[:, idx].cpu(), sel[:, idx], cnt[:, idx],
                            imp[:, idx], out[:, idx], range(Hkv), tol)
    assert rep.compared == B * len(idx) * Hkv and rep.imp_levels > 0, rep
