"""Thin Python binding of librecsa.so (ctypes).

Argument marshalling only: every step of the RecSA path runs in the HIP
kernels behind the C ABI declared in include/recsa.h.  PyTorch provides device
memory and streams.  If the shared library is missing, importing the binding
works but every call raises: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librecsa.so")

RECSA_OK = 0
RECSA_E_INVALID = -1
RECSA_E_UNSUPPORTED = -2
RECSA_E_WORKSPACE = -3
RECSA_E_HIP = -4
RECSA_F32 = 0
RECSA_BF16 = 1
RECSA_MAX_LEVELS = 8

EXPORTS = (
    "recsa_status_string", "recsa_level_rows", "recsa_levels_needed",
    "recsa_init_rope", "recsa_workspace_bytes", "recsa_build_tree",
    "recsa_append_decode", "recsa_select", "recsa_attn_decode",
    "recsa_attn_prefill", "recsa_decode", "recsa_decode_static",
    "recsa_distill_workspace_bytes",
    "recsa_distill_kl", "recsa_shift_workspace_bytes", "recsa_shift_penalty",
    "recsa_pooler_backward_workspace_bytes", "recsa_pooler_backward",
    "recsa_distill_key_grad_workspace_bytes", "recsa_distill_key_grad",
)


class RecsaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class TreeC(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("d", ctypes.c_int32), ("C", ctypes.c_int32), ("k", ctypes.c_int32),
        ("n_levels", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("L_cap", ctypes.c_int64),
        ("K", ctypes.c_void_p * RECSA_MAX_LEVELS),
        ("V", ctypes.c_void_p * RECSA_MAX_LEVELS),
        ("Kr", ctypes.c_void_p * RECSA_MAX_LEVELS),
        ("rope", ctypes.c_void_p),
    ]


class PoolerC(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("hidden", ctypes.c_int32), ("tau", ctypes.c_float),
        ("g", ctypes.c_float), ("eps", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("w", ctypes.c_void_p), ("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
        ("W2", ctypes.c_void_p),
    ]


class PoolerGradC(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("W2", ctypes.c_void_p), ("tau", ctypes.c_void_p), ("g", ctypes.c_void_p)]


_lib = None


def lib():
    """Load librecsa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m long_context_kv_amd.build_lib` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        T, P = ctypes.POINTER(TreeC), ctypes.POINTER(PoolerC)
        sig = {
            "recsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "recsa_level_rows": (i64, [i64, i32, i32]),
            "recsa_levels_needed": (i32, [i64, i32, i32]),
            "recsa_init_rope": (ctypes.c_int, [vp, i32, i32, ctypes.c_double, vp]),
            "recsa_workspace_bytes": (sz, [T, i32, i64]),
            "recsa_build_tree": (ctypes.c_int, [T, P, i64, i64, vp]),
            "recsa_append_decode": (ctypes.c_int, [T, P, vp, vp, vp, vp]),
            "recsa_select": (ctypes.c_int, [T, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "recsa_attn_decode": (ctypes.c_int, [T, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
            "recsa_attn_prefill": (ctypes.c_int, [T, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "recsa_decode": (ctypes.c_int, [T, P, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
            "recsa_decode_static": (ctypes.c_int, [T, P, vp, vp, vp, i32, vp, vp, vp, vp, vp]),
            "recsa_distill_workspace_bytes": (sz, [T, i32, i64]),
            "recsa_distill_kl": (ctypes.c_int, [T, vp, i32, i32, vp, vp, vp, vp,
                                                 ctypes.c_double, vp, vp, vp, sz, vp]),
            "recsa_shift_workspace_bytes": (sz, [T]),
            "recsa_shift_penalty": (ctypes.c_int, [T, P, i64, vp, vp, sz, vp]),
            "recsa_pooler_backward_workspace_bytes": (sz, [T, P, i32]),
            "recsa_distill_key_grad_workspace_bytes": (sz, [T, i32, i64]),
            "recsa_distill_key_grad": (ctypes.c_int, [T, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz,
                                                       vp, vp, sz, vp]),
            "recsa_pooler_backward": (ctypes.c_int, [T, P, i32, i64, vp, vp, ctypes.c_float,
                                                      ctypes.POINTER(PoolerGradC), vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


_hip = None


def host_device_pointer(t: torch.Tensor) -> int:
    """Device address of a pinned host tensor (hipHostGetDevicePointer).
    Raises unless the memory is page-locked host memory that the device can
    address, so no kernel is ever handed an unmapped host pointer."""
    global _hip
    if t.device.type != "cpu" or not t.is_pinned():
        raise ValueError("expected a pinned host tensor")
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipHostGetDevicePointer.restype = ctypes.c_int
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                 ctypes.c_void_p, ctypes.c_uint]
    dp = ctypes.c_void_p()
    err = _hip.hipHostGetDevicePointer(ctypes.byref(dp), ctypes.c_void_p(t.data_ptr()), 0)
    if err != 0 or not dp.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({err}): host memory not mapped")
    return int(dp.value)


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != RECSA_OK:
        raise RecsaError(fn, status, recsa_status_string(status))


# ------------------------------------------------------------ device plumbing

@dataclass
class Tree:
    """One layer's KV tree in device memory (torch tensors) plus its C view.

    K[l], V[l]: [B, Hkv, floor(L_cap / 16^l), d] in the storage dtype; level 0
    is the KV cache itself (pre-RoPE keys).  Kr[l]: the same shape, the rotated
    keys the library writes next to every key row -- or, with
    rotated_keys=False, empty tensors (passed as NULL: the kernels then rotate
    the key rows they read, with the same bits).  rope: [C*k, d/2, 2]
    float32.  With level0_host, K[0], V[0] and Kr[0] are pinned host tensors
    that the kernels read and write in place over PCIe (level0_dptr holds
    their device addresses); levels >= 1 stay in device memory."""
    B: int
    Hkv: int
    d: int
    L_cap: int
    k: int
    C: int
    dtype: str
    n_levels: int
    K: list
    V: list
    Kr: list
    rope: torch.Tensor
    level0_dptr: tuple | None = None

    @staticmethod
    def allocate(B, Hkv, d, L_cap, k=256, C=16, dtype="bf16", n_levels=None,
                 device="cuda", theta=1e6, level0=None, level0_host=False,
                 rotated_keys=True):
        n = n_levels or max(2, recsa_levels_needed(L_cap, C, k))
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        K, V, Kr = [], [], []
        for lvl in range(n):
            rows = recsa_level_rows(L_cap, C, lvl)
            kr_rows = rows if rotated_keys else 0
            if lvl == 0 and level0_host:
                pin = lambda r: torch.zeros((B, Hkv, r, d), dtype=tdt, pin_memory=True)
                Kr.append(pin(kr_rows))
                K.append(pin(rows))
                V.append(pin(rows))
                if level0 is not None:
                    K[0].copy_(level0[0])
                    V[0].copy_(level0[1])
                continue
            Kr.append(torch.zeros((B, Hkv, kr_rows, d), dtype=tdt, device=device))
            if lvl == 0 and level0 is not None:
                K.append(level0[0])
                V.append(level0[1])
                continue
            K.append(torch.zeros((B, Hkv, rows, d), dtype=tdt, device=device))
            V.append(torch.zeros((B, Hkv, rows, d), dtype=tdt, device=device))
        rope = torch.empty((C * k, d // 2, 2), dtype=torch.float32, device=device)
        recsa_init_rope(rope, d, C * k, theta)
        dptr = None
        if level0_host:
            dptr = tuple(host_device_pointer(x) if x.numel() else None for x in (K[0], V[0], Kr[0]))
        return Tree(B, Hkv, d, L_cap, k, C, dtype, n, K, V, Kr, rope, dptr)

    def c(self) -> TreeC:
        t = TreeC()
        t.dtype = RECSA_BF16 if self.dtype == "bf16" else RECSA_F32
        t.B, t.Hkv, t.d, t.C, t.k = self.B, self.Hkv, self.d, self.C, self.k
        t.n_levels, t.L_cap = self.n_levels, self.L_cap
        for lvl in range(self.n_levels):
            t.K[lvl] = self.K[lvl].data_ptr() if self.K[lvl].numel() else None
            t.V[lvl] = self.V[lvl].data_ptr() if self.V[lvl].numel() else None
            t.Kr[lvl] = self.Kr[lvl].data_ptr() if self.Kr[lvl].numel() else None
        if self.level0_dptr is not None:
            t.K[0], t.V[0], t.Kr[0] = self.level0_dptr
        t.rope = self.rope.data_ptr()
        return t

    @property
    def n_sel(self) -> int:
        return max(self.n_levels - 1, 1)

    def selection_buffers(self, n_queries: int, with_importance=False):
        dev = self.rope.device
        sel = torch.full((n_queries, self.Hkv, self.n_sel, self.k), -1,
                         dtype=torch.int32, device=dev)
        cnt = torch.zeros((n_queries, self.Hkv, self.n_sel), dtype=torch.int32, device=dev)
        imp = (torch.zeros((n_queries, self.Hkv, self.n_sel, self.C * self.k),
                           dtype=torch.float32, device=dev) if with_importance else None)
        return sel, cnt, imp


@dataclass
class Pooler:
    """Pooler weights (Eq. 5) as float32 device tensors."""
    w: torch.Tensor
    W1: torch.Tensor
    b1: torch.Tensor
    W2: torch.Tensor
    tau: float
    g: float
    eps: float = 1e-6

    @staticmethod
    def from_dict(p: dict, device="cuda"):
        f = lambda x: x.to(device=device, dtype=torch.float32).contiguous()
        return Pooler(f(p["w"]), f(p["W1"]), f(p["b1"]), f(p["W2"]),
                      float(p["tau"]), float(p["g"]), float(p.get("eps", 1e-6)))

    def c(self) -> PoolerC:
        P = PoolerC()
        P.d, P.hidden = self.w.shape[0], self.W1.shape[0]
        P.tau, P.g, P.eps = self.tau, self.g, self.eps
        P.w, P.W1 = self.w.data_ptr(), self.W1.data_ptr()
        P.b1, P.W2 = self.b1.data_ptr(), self.W2.data_ptr()
        return P


def _tc(tree):
    return tree.c() if isinstance(tree, Tree) else tree


def _pc(p):
    return p.c() if isinstance(p, Pooler) else p


# ------------------------------------------------------------ C ABI mirrors

def recsa_status_string(status: int) -> str:
    return lib().recsa_status_string(status).decode()


def recsa_level_rows(L_cap: int, C: int, level: int) -> int:
    return int(lib().recsa_level_rows(L_cap, C, level))


def recsa_levels_needed(L_cap: int, C: int, k: int) -> int:
    return int(lib().recsa_levels_needed(L_cap, C, k))


def recsa_init_rope(table, d: int, n_pos: int, theta: float, stream=None):
    _check("recsa_init_rope", lib().recsa_init_rope(_ptr(table), d, n_pos, theta, _stream(stream)))


def recsa_workspace_bytes(tree, Hq: int, n_queries: int) -> int:
    tc = _tc(tree)
    return int(lib().recsa_workspace_bytes(ctypes.byref(tc), Hq, n_queries))


def recsa_build_tree(tree, pooler, tok_begin: int, tok_end: int, stream=None):
    tc, pc = _tc(tree), _pc(pooler)
    _check("recsa_build_tree", lib().recsa_build_tree(
        ctypes.byref(tc), ctypes.byref(pc), tok_begin, tok_end, _stream(stream)))


def recsa_append_decode(tree, pooler, k_new, v_new, pos_dev, stream=None):
    tc, pc = _tc(tree), _pc(pooler)
    _check("recsa_append_decode", lib().recsa_append_decode(
        ctypes.byref(tc), ctypes.byref(pc), _ptr(k_new), _ptr(v_new), _ptr(pos_dev),
        _stream(stream)))


def recsa_select(tree, q, Hq: int, T: int, pos_dev, sel_idx, sel_cnt, importance,
                 ws, ws_bytes: int | None = None, stream=None):
    tc = _tc(tree)
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("recsa_select", lib().recsa_select(
        ctypes.byref(tc), _ptr(q), Hq, T, _ptr(pos_dev), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(importance), _ptr(ws), nb, _stream(stream)))


def recsa_attn_decode(tree, q, Hq: int, pos_dev, sel_idx, sel_cnt, out, ws,
                      ws_bytes: int | None = None, stream=None):
    tc = _tc(tree)
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("recsa_attn_decode", lib().recsa_attn_decode(
        ctypes.byref(tc), _ptr(q), Hq, _ptr(pos_dev), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(out), _ptr(ws), nb, _stream(stream)))


def recsa_attn_prefill(tree, q, Hq: int, T: int, pos_dev, sel_idx, sel_cnt, out, ws,
                       ws_bytes: int | None = None, stream=None):
    tc = _tc(tree)
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("recsa_attn_prefill", lib().recsa_attn_prefill(
        ctypes.byref(tc), _ptr(q), Hq, T, _ptr(pos_dev), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(out), _ptr(ws), nb, _stream(stream)))


def recsa_decode(tree, pooler, k_new, v_new, q, Hq: int, pos_dev, sel_idx, sel_cnt, out, ws,
                 ws_bytes: int | None = None, stream=None):
    tc, pc = _tc(tree), _pc(pooler)
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("recsa_decode", lib().recsa_decode(
        ctypes.byref(tc), ctypes.byref(pc), _ptr(k_new), _ptr(v_new), _ptr(q), Hq, _ptr(pos_dev),
        _ptr(sel_idx), _ptr(sel_cnt), _ptr(out), _ptr(ws), nb, _stream(stream)))


def recsa_decode_static(tree, pooler, k_new, v_new, q, Hq: int, pos_dev, sel_idx, sel_cnt, out,
                        stream=None):
    tc, pc = _tc(tree), _pc(pooler)
    _check("recsa_decode_static", lib().recsa_decode_static(
        ctypes.byref(tc), ctypes.byref(pc), _ptr(k_new), _ptr(v_new), _ptr(q), Hq, _ptr(pos_dev),
        _ptr(sel_idx), _ptr(sel_cnt), _ptr(out), _stream(stream)))


def recsa_distill_workspace_bytes(tree, Hq: int, n_queries: int) -> int:
    tc = _tc(tree)
    return int(lib().recsa_distill_workspace_bytes(ctypes.byref(tc), Hq, n_queries))


def recsa_distill_kl(tree, q, Hq: int, T: int, pos_dev, sel_idx, sel_cnt, importance,
                     theta: float, kl_out, ws, ws_bytes: int | None = None, stream=None,
                     teacher=None):
    tc = _tc(tree)
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("recsa_distill_kl", lib().recsa_distill_kl(
        ctypes.byref(tc), _ptr(q), Hq, T, _ptr(pos_dev), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(importance), theta, _ptr(kl_out), _ptr(teacher), _ptr(ws), nb, _stream(stream)))


def recsa_shift_workspace_bytes(tree) -> int:
    tc = _tc(tree)
    return int(lib().recsa_shift_workspace_bytes(ctypes.byref(tc)))


def recsa_shift_penalty(tree, pooler, tok_end: int, out, ws, ws_bytes: int | None = None,
                        stream=None):
    tc, pc = _tc(tree), _pc(pooler)
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("recsa_shift_penalty", lib().recsa_shift_penalty(
        ctypes.byref(tc), ctypes.byref(pc), tok_end, _ptr(out), _ptr(ws), nb, _stream(stream)))


def recsa_pooler_backward_workspace_bytes(tree, pooler, level: int) -> int:
    tc, pc = _tc(tree), _pc(pooler)
    return int(lib().recsa_pooler_backward_workspace_bytes(ctypes.byref(tc), ctypes.byref(pc),
                                                           level))


def recsa_distill_key_grad_workspace_bytes(tree, Hq: int, n_queries: int) -> int:
    tc = _tc(tree)
    return int(lib().recsa_distill_key_grad_workspace_bytes(ctypes.byref(tc), Hq, n_queries))


def key_grad_buffer(tree):
    """Zeroed float32 buffer for recsa_distill_key_grad's output and the
    per-level views [B, Hkv, rows_l, d] into it (level l at index l - 1)."""
    sizes = [tree.B * tree.Hkv * recsa_level_rows(tree.L_cap, tree.C, l) * tree.d
             for l in range(1, tree.n_levels)]
    buf = torch.zeros(max(sum(sizes), 1), dtype=torch.float32, device=tree.rope.device)
    views, off = [], 0
    for l, n in zip(range(1, tree.n_levels), sizes):
        views.append(buf[off:off + n].view(tree.B, tree.Hkv, -1, tree.d))
        off += n
    return buf, views


def recsa_distill_key_grad(tree, q, Hq: int, T: int, pos_dev, sel_idx, sel_cnt, importance,
                           teacher, select_ws, dK_out, ws, ws_bytes: int | None = None,
                           stream=None):
    tc = _tc(tree)
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    sb = select_ws.numel() * select_ws.element_size()
    _check("recsa_distill_key_grad", lib().recsa_distill_key_grad(
        ctypes.byref(tc), _ptr(q), Hq, T, _ptr(pos_dev), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(importance), _ptr(teacher), _ptr(select_ws), sb, _ptr(dK_out), _ptr(ws), nb,
        _stream(stream)))


def pooler_grad_buffers(pooler) -> dict:
    """Zeroed float32 gradient arrays shaped like the pooler's parameters."""
    dev = pooler.w.device
    return {"w": torch.zeros_like(pooler.w), "W1": torch.zeros_like(pooler.W1),
            "b1": torch.zeros_like(pooler.b1), "W2": torch.zeros_like(pooler.W2),
            "tau": torch.zeros(1, dtype=torch.float32, device=dev),
            "g": torch.zeros(1, dtype=torch.float32, device=dev)}


def recsa_pooler_backward(tree, pooler, level: int, tok_end: int, dK, shift_sums,
                          shift_weight: float, grad: dict, ws, ws_bytes: int | None = None,
                          stream=None):
    tc, pc = _tc(tree), _pc(pooler)
    gc = PoolerGradC(*(grad[n].data_ptr() for n in ("w", "W1", "b1", "W2", "tau", "g")))
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("recsa_pooler_backward", lib().recsa_pooler_backward(
        ctypes.byref(tc), ctypes.byref(pc), level, tok_end, _ptr(dK), _ptr(shift_sums),
        float(shift_weight), ctypes.byref(gc), _ptr(ws), nb, _stream(stream)))


def workspace(tree, Hq: int, n_queries: int):
    """Allocate a zero-filled workspace of the size recsa_workspace_bytes
    reports (zero control words, as recsa_decode requires on first use)."""
    nb = recsa_workspace_bytes(tree, Hq, n_queries)
    if nb == 0:
        raise RecsaError("recsa_workspace_bytes", RECSA_E_INVALID, "invalid arguments")
    return torch.zeros(nb, dtype=torch.uint8, device=tree.rope.device)


CTL_WORDS = 16 + 16 * 32      # per (sequence, KV head): see recsa_decode in recsa.h


def decode_error_words(ws, tree, Hq: int):
    """Error words of the fused-decode control blocks, one per (sequence, KV
    head); nonzero means that group gave up waiting (its output is NaN)."""
    nb = recsa_workspace_bytes(tree, Hq, tree.B)
    n = tree.B * tree.Hkv
    ctl = ws[nb - 4 * CTL_WORDS * n: nb].view(torch.int32).view(n, CTL_WORDS)
    return ctl[:, 1]


def decode_control_words(ws, tree, Hq: int):
    """The whole fused-decode control block [B*Hkv, CTL_WORDS] (int32)."""
    nb = recsa_workspace_bytes(tree, Hq, tree.B)
    n = tree.B * tree.Hkv
    return ws[nb - 4 * CTL_WORDS * n: nb].view(torch.int32).view(n, CTL_WORDS)
