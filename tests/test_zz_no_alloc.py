"""recsa_decode_static (the allocation-free decode) against recsa_decode on
the same inputs, through the C ABI: two calls in a row, the second on a
smaller tree, each giving the existing entry point's selection and output
bit for bit (same kernels, same launch shape); its control words start
clean every call."""

import numpy as np
import pytest
import torch

import synth
from tests.test_gpu_parity import DEV, _need_gpu, _setup

pytestmark = pytest.mark.gpu

R = pytest.importorskip("long_context_kv_amd.recsa")


def _one(B, Hkv, G, d, L, k, dtype, seed):
    Hq = Hkv * G
    L_cap = L + 64
    wl, tree, pool, pdict = _setup(B, Hkv, d, L + 1, L_cap, k, dtype, seed)
    ref = R.Tree.allocate(B, Hkv, d, L_cap, k=k, dtype=dtype, device=DEV,
                          level0=(tree.K[0].clone(), tree.V[0].clone()))
    kn, vn = tree.K[0][:, :, L].clone().contiguous(), tree.V[0][:, :, L].clone().contiguous()
    R.recsa_build_tree(tree, pool, 0, L)
    R.recsa_build_tree(ref, pool, 0, L)
    q = synth.to_storage(synth.normal((B, 1, Hq, d), DEV, seed, 77), dtype)
    pos = torch.full((B,), L, dtype=torch.int64, device=DEV)
    sel, cnt, _ = tree.selection_buffers(B)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    print(f"no-alloc decode: B={B} Hkv={Hkv} G={G} d={d} {dtype} t={L}", flush=True)
    R.recsa_decode_static(tree, pool, kn, vn, q, Hq, pos, sel, cnt, out)
    ws = R.workspace(ref, Hq, B)
    s2, c2, _ = ref.selection_buffers(B)
    o2 = torch.empty_like(out)
    R.recsa_decode(ref, pool, kn, vn, q, Hq, pos, s2, c2, o2, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel, s2) and torch.equal(cnt, c2)
    assert torch.isfinite(out).all()
    assert torch.equal(out, o2)
    for lvl in range(tree.n_levels):
        assert torch.equal(tree.K[lvl], ref.K[lvl]) and torch.equal(tree.Kr[lvl], ref.Kr[lvl])


def test_static_decode_equals_decode_twice_second_smaller():
    _need_gpu()
    _one(2, 8, 4, 128, 65536 + 15, 256, "bf16", 91)      # two scored levels
    _one(1, 2, 2, 64, 5000, 16, "bf16", 92)              # smaller: fewer groups, d = 64
