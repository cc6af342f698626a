"""The fused decode's device-wide barrier form (per-workgroup flags with
device-scope atomics and release/acquire fences), which a device other than
gfx950, or RECSA_FUSED_XCD_LOCAL=0, selects instead of the XCD-local form.
The library picks the form once per process, so the check runs in a fresh
child process with the variable set before its first GPU call: the fused step
must give the separate calls' selection bit for bit and their output to
float32 rounding (the partial softmax states are split differently), match the
oracle, and leave its control words zero."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys
sys.path.insert(0, ROOT)
import numpy as np
import torch
import synth
from long_context_kv_amd import recsa as R
from tests import test_gpu_parity as TP
from tests.test_gpu_parity import DEV

print("device-wide barrier: fused decode vs separate calls vs oracle", flush=True)
B, Hkv, d, k, G = 2, 4, 128, 64, 4
L = 40000
wl, tree, pool, pdict = TP._setup(B, Hkv, d, L + 1, L + 64, k, "bf16", 55)
ref = R.Tree.allocate(B, Hkv, d, L + 64, k=k, dtype="bf16", device=DEV,
                      level0=(tree.K[0].clone(), tree.V[0].clone()))
kn = tree.K[0][:, :, L].clone().contiguous()
vn = tree.V[0][:, :, L].clone().contiguous()
R.recsa_build_tree(tree, pool, 0, L)
R.recsa_build_tree(ref, pool, 0, L)
Hq = Hkv * G
q = synth.to_storage(synth.normal((B, 1, Hq, d), DEV, 55, 9), "bf16")
pos = torch.full((B,), L, dtype=torch.int64, device=DEV)
for rep in range(3):
    sel, cnt, out, ws = TP._fused_step(tree, pool, kn, vn, q, Hq, pos)
    torch.cuda.synchronize()
    assert torch.count_nonzero(R.decode_control_words(ws, tree, Hq)).item() == 0, rep
R.recsa_append_decode(ref, pool, kn, vn, pos)
s2, c2, m2, o2 = TP._run_select_attn(ref, q, Hq, pos.view(B, 1), decode=True)
assert np.array_equal(sel.cpu().numpy().reshape(s2.shape), s2)
o = out.cpu().numpy().astype(np.float64).reshape(o2.shape)
assert np.allclose(o, o2, rtol=0, atol=1e-5 * np.abs(o2).max())   # other partial split
rp = TP._check_queries(ref, pdict, q, pos.view(B, 1).cpu(), s2, c2, m2, o2, range(Hkv), 2e-3)
assert rp.compared == B * Hkv, rp
print("device-wide barrier: ok", flush=True)
'''


def test_fused_decode_device_wide_barrier_in_child_process():
    env = dict(os.environ, RECSA_FUSED_XCD_LOCAL="0")
    r = subprocess.run([sys.executable, "-c", CHILD.replace("ROOT", repr(ROOT))], env=env,
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "device-wide barrier: ok" in r.stdout
