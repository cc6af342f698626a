"""Host-side checks of librecsa.so that need no GPU: every symbol declared in
include/recsa.h is exported, the layout helpers are right, and argument
validation rejects bad calls with the documented status before launching."""

import ctypes
import os
import re

import pytest

from long_context_kv_amd import recsa as R

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "recsa.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(recsa_\w+)\s*\(", txt, re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("recsa_build_tree", "recsa_append_decode", "recsa_select",
              "recsa_attn_decode", "recsa_attn_prefill"):
        assert n in names
    assert set(names) == set(R.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(R.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n


def test_layout_helpers():
    assert R.recsa_level_rows(524288, 16, 0) == 524288
    assert R.recsa_level_rows(524288, 16, 2) == 2048
    assert R.recsa_level_rows(100, 16, 2) == 0
    assert R.recsa_levels_needed(4096, 16, 16) == 3          # tiny workload: 3 levels
    assert R.recsa_levels_needed(524288 + 4096, 16, 256) == 4
    assert R.recsa_levels_needed(1048577, 16, 256) == 5
    assert R.recsa_levels_needed(256, 16, 256) == 1
    assert R.recsa_status_string(R.RECSA_E_WORKSPACE) == "workspace too small"
    assert R.recsa_status_string(12345) == "unknown status"


def _tree(**over):
    t = R.TreeC()
    t.dtype, t.B, t.Hkv, t.d, t.C, t.k = R.RECSA_BF16, 1, 8, 128, 16, 256
    t.L_cap, t.n_levels = 528384, 4
    for lvl in range(4):
        t.K[lvl] = 0x1000 * (lvl + 1)       # never dereferenced: validation fails first
        t.V[lvl] = 0x2000 * (lvl + 1)
        t.Kr[lvl] = 0x5000 * (lvl + 1)
    t.rope = 0x3000
    for k, v in over.items():
        setattr(t, k, v)
    return t


def _pooler(**over):
    p = R.PoolerC()
    p.d, p.hidden, p.tau, p.g, p.eps = 128, 128, 1.0, 0.5, 1e-6
    p.w = p.W1 = p.b1 = p.W2 = 0x4000
    for k, v in over.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("over,status", [
    (dict(C=8), R.RECSA_E_UNSUPPORTED),
    (dict(d=96), R.RECSA_E_UNSUPPORTED),
    (dict(k=513), R.RECSA_E_UNSUPPORTED),      # C*k above 8192
    (dict(dtype=7), R.RECSA_E_UNSUPPORTED),
    (dict(n_levels=3), R.RECSA_E_INVALID),      # top list would exceed k
    (dict(n_levels=9), R.RECSA_E_INVALID),
    (dict(B=0), R.RECSA_E_INVALID),
    (dict(rope=None), R.RECSA_E_INVALID),
])
def test_tree_validation(over, status):
    L = R.lib()
    t = _tree(**over)
    p = _pooler()
    assert L.recsa_build_tree(ctypes.byref(t), ctypes.byref(p), 0, 16, None) == status


def test_k512_is_accepted():
    """k = 512 (C*k = 8192 list positions) is a supported selection depth:
    validation passes and the workspace holds 8192 logits per scored level."""
    L = R.lib()
    t = _tree(k=512)
    a = L.recsa_workspace_bytes(ctypes.byref(t), 32, 1)
    b = L.recsa_workspace_bytes(ctypes.byref(t), 32, 2)
    assert a > 0 and b - a >= 8 * (3 * 4 * 8192 * 4 + 3 * 256 * 4)


def test_call_validation_without_launch():
    L = R.lib()
    t, p = _tree(), _pooler()
    b = ctypes.byref
    assert L.recsa_build_tree(None, b(p), 0, 16, None) == R.RECSA_E_INVALID
    assert L.recsa_build_tree(b(t), b(p), 0, t.L_cap + 1, None) == R.RECSA_E_INVALID
    assert L.recsa_build_tree(b(t), b(p), 10, 5, None) == R.RECSA_E_INVALID
    assert L.recsa_build_tree(b(t), b(p), 7, 7, None) == R.RECSA_OK          # empty range
    t_nokr = _tree()
    t_nokr.Kr[1] = None
    assert L.recsa_build_tree(b(t_nokr), b(p), 0, 16, None) == R.RECSA_E_INVALID
    assert L.recsa_build_tree(b(t), b(_pooler(d=64)), 0, 16, None) == R.RECSA_E_INVALID
    assert L.recsa_build_tree(b(t), b(_pooler(hidden=100)), 0, 16, None) == R.RECSA_E_INVALID
    assert L.recsa_build_tree(b(t), b(_pooler(eps=-1.0)), 0, 16, None) == R.RECSA_E_INVALID
    assert L.recsa_append_decode(b(t), b(p), None, 0x10, 0x10, None) == R.RECSA_E_INVALID
    ws_need = L.recsa_workspace_bytes(b(t), 32, 1)
    assert ws_need > 0
    assert L.recsa_workspace_bytes(b(t), 30, 1) == 0                        # Hq % Hkv
    args = (b(t), 0x10, 32, 1, 0x10, 0x10, 0x10, None, 0x10)
    assert L.recsa_select(*args, ws_need - 1, None) == R.RECSA_E_WORKSPACE
    assert L.recsa_select(b(t), 0x10, 24, 1, 0x10, 0x10, 0x10, None, 0x10, ws_need, None) \
        == R.RECSA_E_UNSUPPORTED                                            # G = 3
    assert L.recsa_select(b(t), 0x10, 64, 1, 0x10, 0x10, 0x10, None, 0x10, ws_need, None) \
        == R.RECSA_E_UNSUPPORTED                                            # G = 8: off
    assert L.recsa_decode(b(t), b(p), 0x10, 0x10, 0x10, 64, 0x10, 0x10, 0x10, 0x10, 0x10,
                          ws_need, None) == R.RECSA_E_UNSUPPORTED
    assert L.recsa_select(b(t), None, 32, 1, 0x10, 0x10, 0x10, None, 0x10, ws_need, None) \
        == R.RECSA_E_INVALID
    assert L.recsa_attn_decode(b(t), 0x10, 32, 0x10, 0x10, 0x10, None, 0x10, ws_need, None) \
        == R.RECSA_E_INVALID
    assert L.recsa_attn_prefill(b(t), 0x10, 32, 0, 0x10, 0x10, 0x10, 0x10, 0x10, ws_need, None) \
        == R.RECSA_E_INVALID
    assert L.recsa_init_rope(None, 128, 4096, 1e6, None) == R.RECSA_E_INVALID
    assert L.recsa_init_rope(0x10, 127, 4096, 1e6, None) == R.RECSA_E_INVALID


def test_workspace_grows_with_queries():
    L = R.lib()
    t = _tree()
    a = L.recsa_workspace_bytes(ctypes.byref(t), 32, 1)
    b = L.recsa_workspace_bytes(ctypes.byref(t), 32, 4096)
    # logits of 3 selection levels x 4 heads x 4096 positions per (query, head),
    # their bitmaps, and (bf16, >= 256 query-head slots) the scoring buckets:
    # one region of 256 queries x k entries (uint2) per filing workgroup
    # (4096/256 + B blocks per KV head) and its tiles (uint4, at most one
    # partial tile per parent of level 1, N_2 + 1 of them), plus the tile
    # count, each region 256-byte aligned
    def al(x):
        return (x + 255) // 256 * 256
    regions = (4096 // 256 + 1) * 8
    n_up = 528384 // 256 + 1
    tiles = regions * (min(n_up, 256 * 256) + 256 * 256 // 64)
    buckets = al(tiles * 16) + al(regions * 256 * 256 * 8) + al(4)
    assert b - a == 4095 * 8 * (3 * 4 * 4096 * 4 + 3 * 128 * 4) + buckets
    # float32 trees are scored per query: no bucket region
    tf = _tree(dtype=R.RECSA_F32)
    af = L.recsa_workspace_bytes(ctypes.byref(tf), 32, 1)
    bf = L.recsa_workspace_bytes(ctypes.byref(tf), 32, 4096)
    assert bf - af == 4095 * 8 * (3 * 4 * 4096 * 4 + 3 * 128 * 4)


def test_distillation_calls_validate_without_launch():
    """The Eq. 6 / Eq. 7 calls: workspace sizes from their documented layout,
    and bad arguments rejected before any launch."""
    L = R.lib()
    b = ctypes.byref
    # a 32K-token tree at k = 64 (4 levels), the pages' pooler-training shape
    t = _tree(k=64, L_cap=32768, n_levels=4)
    p = _pooler()
    def al(x):
        return (x + 255) // 256 * 256
    need = L.recsa_distill_workspace_bytes(b(t), 32, 100)
    assert need == al(32768 * 128 * 4) + al(8 * 32768 * 128 * 4) + 100 * 32 * (32768 // 16) * 4
    assert L.recsa_distill_workspace_bytes(b(t), 30, 100) == 0              # Hq % Hkv
    # ceil(L_cap/16) + C*k > 16376: the per-query masses no longer fit on chip
    big = _tree(k=256, L_cap=528384, n_levels=4)
    assert L.recsa_distill_workspace_bytes(b(big), 32, 1) == 0
    args = [b(big), 0x10, 32, 1, 0x10, 0x10, 0x10, 0x10, 1e6, 0x10, None, 0x10, 1 << 40, None]
    assert L.recsa_distill_kl(*args) == R.RECSA_E_UNSUPPORTED
    ok = [b(t), 0x10, 32, 100, 0x10, 0x10, 0x10, 0x10, 1e6, 0x10, None, 0x10, need, None]
    for i in (1, 4, 5, 6, 7, 9, 11):                      # required pointers
        a = list(ok)
        a[i] = None
        assert L.recsa_distill_kl(*a) == R.RECSA_E_INVALID, i
    a = list(ok)
    a[8] = 1.0                                            # theta must exceed 1
    assert L.recsa_distill_kl(*a) == R.RECSA_E_INVALID
    a = list(ok)
    a[12] = need - 1
    assert L.recsa_distill_kl(*a) == R.RECSA_E_WORKSPACE
    a = list(ok)
    a[2] = 24                                             # G = 3
    assert L.recsa_distill_kl(*a) == R.RECSA_E_UNSUPPORTED
    # shift penalty: one partial row of d+1 floats per 16 nodes, every level
    sw = L.recsa_shift_workspace_bytes(b(t))
    rows = sum((32768 // 16 ** lvl + 15) // 16 for lvl in (1, 2, 3)) * 8
    assert sw == rows * 129 * 4
    assert L.recsa_shift_penalty(b(t), b(p), 0, 0x10, 0x10, sw, None) == R.RECSA_E_INVALID
    assert L.recsa_shift_penalty(b(t), b(p), 32769, 0x10, 0x10, sw, None) == R.RECSA_E_INVALID
    assert L.recsa_shift_penalty(b(t), b(p), 4096, None, 0x10, sw, None) == R.RECSA_E_INVALID
    assert L.recsa_shift_penalty(b(t), b(p), 4096, 0x10, 0x10, sw - 1, None) \
        == R.RECSA_E_WORKSPACE
    assert L.recsa_shift_penalty(b(t), b(_pooler(d=64)), 4096, 0x10, 0x10, sw, None) \
        == R.RECSA_E_INVALID


def test_pooler_backward_validates_without_launch():
    L = R.lib()
    b = ctypes.byref
    t = _tree(k=64, L_cap=32768, n_levels=4)
    p = _pooler()
    need = L.recsa_pooler_backward_workspace_bytes(b(t), b(p), 1)
    # one row of 3d + 2*hidden floats per node slot (16 per tile), then d+2
    # floats per tile, then one float64 partial of every gradient element per
    # 512 node slots, each region 256-byte aligned
    al = lambda x: (x + 255) // 256 * 256
    tiles = (2048 + 15) // 16 * 8
    rows = tiles * 16 * (3 * 128 + 2 * 128) * 4
    outputs = 128 * 3 * 128 + 128 + 128 + 2
    assert need == al(rows) + al(tiles * 130 * 4) + (tiles * 16 // 512) * outputs * 8
    assert L.recsa_pooler_backward_workspace_bytes(b(t), b(p), 0) == 0    # level >= 1
    assert L.recsa_pooler_backward_workspace_bytes(b(t), b(p), 4) == 0    # level < n_levels
    g = R.PoolerGradC(0x10, 0x10, 0x10, 0x10, 0x10, 0x10)
    ok = [b(t), b(p), 1, 4096, 0x10, 0x10, 0.5, b(g), 0x10, need, None]
    for i, bad in ((2, 0), (2, 4), (3, 0), (3, 32769), (8, None)):
        a = list(ok)
        a[i] = bad
        assert L.recsa_pooler_backward(*a) == R.RECSA_E_INVALID, (i, bad)
    a = list(ok)
    a[6] = float("inf")
    assert L.recsa_pooler_backward(*a) == R.RECSA_E_INVALID
    a = list(ok)
    a[9] = need - 1
    assert L.recsa_pooler_backward(*a) == R.RECSA_E_WORKSPACE
    g_missing = R.PoolerGradC(0x10, None, 0x10, 0x10, 0x10, 0x10)
    a = list(ok)
    a[7] = b(g_missing)
    assert L.recsa_pooler_backward(*a) == R.RECSA_E_INVALID


def test_key_grad_validates_without_launch():
    """recsa_distill_key_grad: workspace size from its documented layout
    (softmax figures, then the per-chunk partial sums of level 1), and bad
    arguments rejected before any launch."""
    L = R.lib()
    b = ctypes.byref
    t = _tree(k=64, L_cap=32768, n_levels=4)
    al = lambda x: (x + 255) // 256 * 256
    nq = 5000
    need = L.recsa_distill_key_grad_workspace_bytes(b(t), 32, nq)
    stats = al(nq * 8 * 3 * 4 * 16)
    parents, chunks = 2048 // 16, (nq + 2047) // 2048
    assert need == stats + 8 * parents * chunks * 16 * 128 * 4
    assert L.recsa_distill_key_grad_workspace_bytes(b(t), 30, nq) == 0     # Hq % Hkv
    assert L.recsa_distill_key_grad_workspace_bytes(b(t), 32, 0) == 0
    sws = L.recsa_workspace_bytes(b(t), 32, nq)
    ok = [b(t), 0x10, 32, nq, 0x10, 0x10, 0x10, 0x10, 0x10, 0x10, sws, 0x10, 0x10, need, None]
    for i in (1, 4, 5, 6, 7, 8, 9, 11, 12):                # required pointers
        a = list(ok)
        a[i] = None
        assert L.recsa_distill_key_grad(*a) == R.RECSA_E_INVALID, i
    a = list(ok)
    a[3] = 0                                              # T >= 1
    assert L.recsa_distill_key_grad(*a) == R.RECSA_E_INVALID
    a = list(ok)
    a[10] = sws - 1
    assert L.recsa_distill_key_grad(*a) == R.RECSA_E_WORKSPACE
    a = list(ok)
    a[13] = need - 1
    assert L.recsa_distill_key_grad(*a) == R.RECSA_E_WORKSPACE
    a = list(ok)
    a[2] = 24                                             # G = 3
    assert L.recsa_distill_key_grad(*a) == R.RECSA_E_UNSUPPORTED


def test_misaligned_arrays_are_rejected_without_launch():
    """Float and bf16 arrays must be 16-byte aligned, index arrays naturally
    aligned; a misaligned pointer is RECSA_E_INVALID before any launch."""
    L = R.lib()
    b = ctypes.byref
    t = _tree()
    need = L.recsa_workspace_bytes(b(t), 32, 1)
    ok = [b(t), 0x10, 32, 1, 0x10, 0x10, 0x10, None, 0x100, need, None]
    for i, bad in ((1, 0x18), (4, 0x14), (5, 0x12), (6, 0x11), (8, 0x108)):
        a = list(ok)
        a[i] = bad
        assert L.recsa_select(*a) == R.RECSA_E_INVALID, (i, bad)
    a = list(ok)
    a[7] = 0x24                                           # importance: 16-byte
    assert L.recsa_select(*a) == R.RECSA_E_INVALID
    mis = _tree()
    mis.Kr[1] = 0x5008
    assert L.recsa_workspace_bytes(b(mis), 32, 1) == 0
    p = _pooler(W1=0x4004)
    assert L.recsa_build_tree(b(t), b(p), 0, 16, None) == R.RECSA_E_INVALID
    assert L.recsa_init_rope(0x3004, 128, 16, 1e6, None) == R.RECSA_E_INVALID


def test_misaligned_distillation_arrays_are_rejected_without_launch():
    """The distillation calls apply the same alignment rule: 16 bytes for
    float arrays, 4 for the per-query KL output and the scalar gradients."""
    L = R.lib()
    b = ctypes.byref
    t = _tree(k=64, L_cap=32768, n_levels=4)
    p = _pooler()
    nq = 100
    dneed = L.recsa_distill_workspace_bytes(b(t), 32, nq)
    ok = [b(t), 0x10, 32, nq, 0x10, 0x10, 0x10, 0x10, 1e6, 0x10, None, 0x10, dneed, None]
    for i, bad in ((1, 0x18), (7, 0x14), (11, 0x108)):
        a = list(ok)
        a[i] = bad
        assert L.recsa_distill_kl(*a) == R.RECSA_E_INVALID, (i, bad)
    a = list(ok)
    a[10] = 0x24                                          # teacher output: 16-byte
    assert L.recsa_distill_kl(*a) == R.RECSA_E_INVALID
    kneed = L.recsa_distill_key_grad_workspace_bytes(b(t), 32, nq)
    sws = L.recsa_workspace_bytes(b(t), 32, nq)
    ok = [b(t), 0x10, 32, nq, 0x10, 0x10, 0x10, 0x10, 0x10, 0x10, sws, 0x10, 0x10, kneed, None]
    for i, bad in ((7, 0x14), (8, 0x18), (9, 0x104), (11, 0x1c), (12, 0x108)):
        a = list(ok)
        a[i] = bad
        assert L.recsa_distill_key_grad(*a) == R.RECSA_E_INVALID, (i, bad)
    bneed = L.recsa_pooler_backward_workspace_bytes(b(t), b(p), 1)
    g = R.PoolerGradC(0x10, 0x10, 0x10, 0x10, 0x14, 0x18)    # scalar gradients: 4-byte
    ok = [b(t), b(p), 1, 4096, 0x10, 0x18, 0.5, b(g), 0x10, bneed, None]
    for i, bad in ((4, 0x14), (5, 0x12), (8, 0x108)):
        a = list(ok)
        a[i] = bad
        assert L.recsa_pooler_backward(*a) == R.RECSA_E_INVALID, (i, bad)
    g_bad = R.PoolerGradC(0x10, 0x18, 0x10, 0x10, 0x14, 0x18)
    a = list(ok)
    a[7] = b(g_bad)
    assert L.recsa_pooler_backward(*a) == R.RECSA_E_INVALID
    # the decode step: q, the new rows, the output and the workspace
    t2 = _tree()
    need = L.recsa_workspace_bytes(b(t2), 32, 1)
    ok = [b(t2), b(p), 0x10, 0x10, 0x10, 32, 0x10, 0x10, 0x10, 0x10, 0x100, need, None]
    for i in (2, 3, 4, 9, 10):
        a = list(ok)
        a[i] = ok[i] + 8
        assert L.recsa_decode(*a) == R.RECSA_E_INVALID, i


def test_static_decode_validation_and_scratch_limit():
    """recsa_decode_static validates like recsa_decode (nothing is launched
    on an error) and rejects configurations whose workspace exceeds its
    32 MiB device array: 8 sequences x 8 KV heads at G = 4, k = 256 and 5
    levels need 25 MiB and pass validation; 16 x 8 need 51 MiB."""
    L = R.lib()
    b = ctypes.byref
    p = _pooler()
    ok = [None, b(p), 0x10, 0x10, 0x10, 32, 0x10, 0x10, 0x10, 0x10, None]
    t = _tree(B=8, L_cap=1 << 20, n_levels=5)
    for lvl in range(5):
        t.K[lvl], t.V[lvl], t.Kr[lvl] = 0x1000 * (lvl + 1), 0x2000 * (lvl + 1), 0x5000 * (lvl + 1)
    need = L.recsa_workspace_bytes(b(t), 32, 8)
    assert 24 << 20 < need <= 32 << 20
    big = _tree(B=16, L_cap=1 << 20, n_levels=5)
    for lvl in range(5):
        big.K[lvl], big.V[lvl], big.Kr[lvl] = t.K[lvl], t.V[lvl], t.Kr[lvl]
    assert L.recsa_workspace_bytes(b(big), 32, 16) > 32 << 20
    a = list(ok)
    a[0] = b(big)
    assert L.recsa_decode_static(*a) == R.RECSA_E_WORKSPACE
    for i, bad in ((2, 0x18), (3, 0x18), (4, 0x18), (6, 0x14), (9, 0x18), (6, None)):
        a = list(ok)
        a[0] = b(_tree())
        a[i] = bad
        assert L.recsa_decode_static(*a) == R.RECSA_E_INVALID, (i, bad)
    a = list(ok)
    a[0], a[5] = b(_tree()), 64                                   # G = 8: off
    assert L.recsa_decode_static(*a) == R.RECSA_E_UNSUPPORTED


def test_rotated_key_copy_is_all_or_nothing():
    """Kr may be absent (every level NULL: the kernels rotate raw key rows),
    but a tree with it at some levels and not at others is invalid."""
    L = R.lib()
    b = ctypes.byref
    p = _pooler()
    none = _tree()
    for lvl in range(4):
        none.Kr[lvl] = None
    # validation passes (an empty token range launches nothing)
    assert L.recsa_build_tree(b(none), b(p), 5, 5, None) == R.RECSA_OK
    assert L.recsa_workspace_bytes(b(none), 32, 1) > 0
    mixed = _tree()
    mixed.Kr[2] = None
    assert L.recsa_build_tree(b(mixed), b(p), 5, 5, None) == R.RECSA_E_INVALID
    mixed0 = _tree()
    mixed0.Kr[0] = None
    assert L.recsa_workspace_bytes(b(mixed0), 32, 1) == 0
