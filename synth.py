"""Seeded synthetic inputs for RecSA workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path (through the tests and the benchmark)
and the CPU oracle consume exactly the tensors it returns.

Workloads (Qwen3-4B-shaped single attention layer unless stated):
  tiny      1 KV head, 4 query heads, d=64,  fp32, L=4096,  C=16, k=16
  131k      8 KV heads, 32 query heads, d=128, bf16, L=131072,  C=16, k=256
  524k      same shape, L=524288, decode batch 1 + a 4096-query prefill chunk
  1m_b4     same shape, L=1048576, decode batch 4 (independent sequences)
  2m_l4     4 layers of the same shape at L=2097152
  distill_32k  same shape at L=32768 with k=64, every position a query

K and V rows are N(0,1); decode queries are N(0,1); 16 "needle" keys per
(sequence, KV head) are planted at uniform random positions, aligned with
cosine 0.9 to the mean direction of that KV head's decode queries.  Pooler
weights are N(0, 1/d), tau=1, g=0.5, eps=1e-6, hidden width h=d; RoPE base
1e6.  All draws come from torch generators seeded per (workload seed, role).
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import torch

ROLE = {"k": 1, "v": 2, "q": 3, "needle": 4, "pooler": 5, "chunk": 6,
        "decode_kv": 7, "needle_pos": 8}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hkv: int
    Hq: int
    d: int
    dtype: str          # 'bf16' | 'f32'
    L: int              # tokens already in the cache
    C: int
    k: int
    seed: int
    n_decode_q: int = 1     # decode queries per sequence (tiny: 8 at the tail)
    prefill_T: int = 0      # prefill chunk length appended at [L, L+T)
    n_needles: int = 16
    n_layers: int = 1
    decode_steps: int = 1
    theta: float = 1e6

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 4, 64, "f32", 4096, 16, 16, 0,
                     n_decode_q=8, n_needles=0),
    "131k": Workload("131k", 1, 8, 32, 128, "bf16", 131072, 16, 256, 1),
    "524k": Workload("524k", 1, 8, 32, 128, "bf16", 524288, 16, 256, 2,
                     prefill_T=4096),
    "1m_b4": Workload("1m_b4", 4, 8, 32, 128, "bf16", 1048576, 16, 256, 3),
    "2m_l4": Workload("2m_l4", 1, 8, 32, 128, "bf16", 2097152, 16, 256, 4,
                      prefill_T=8192, n_layers=4, decode_steps=256),
    # pooler distillation at the training length: every position of a
    # 32768-token sequence is a query, k = 64
    "distill_32k": Workload("distill_32k", 1, 8, 32, 128, "bf16", 32768, 16, 64, 5,
                            n_needles=0),
}


def seed_for(*parts) -> int:
    """Stable 63-bit seed from a tuple of ints/strings."""
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def generator(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*parts))
    return g


def normal(shape, device, *parts, std=1.0):
    """N(0, std^2) float32 tensor from a CPU generator seeded by ``parts``,
    moved to ``device`` (so every device sees the same numbers)."""
    g = generator("cpu", *parts)
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(device)


def to_storage(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round-to-nearest-even into the storage dtype."""
    return x.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def pooler_params(d: int, h: int, device, seed: int, layer: int = 0):
    """Pooler weights of the workloads: w, W1, b1, W2 ~ N(0, 1/d)."""
    std = d ** -0.5
    return dict(
        w=normal((d,), device, seed, ROLE["pooler"], layer, 0, std=std),
        W1=normal((h, 2 * d), device, seed, ROLE["pooler"], layer, 1, std=std),
        b1=normal((h,), device, seed, ROLE["pooler"], layer, 2, std=std),
        W2=normal((d, h), device, seed, ROLE["pooler"], layer, 3, std=std),
        tau=1.0, g=0.5, eps=1e-6,
    )


def decode_queries(wl: Workload, device, step: int = 0, layer: int = 0):
    """[B, n_decode_q, Hq, d] queries in the storage dtype."""
    q = normal((wl.B, wl.n_decode_q, wl.Hq, wl.d), device, wl.seed, ROLE["q"],
               layer, step)
    return to_storage(q, wl.dtype)


def kv_rows(wl: Workload, device, layer: int = 0, n_rows: int | None = None,
            b_list=None, h_list=None):
    """Level-0 K and V [B, Hkv, n_rows, d] in the storage dtype.

    Rows are drawn per (sequence, KV head) so that any subset of heads can be
    regenerated on its own (the CPU oracle uses that)."""
    n = wl.L if n_rows is None else n_rows
    bs = range(wl.B) if b_list is None else b_list
    hs = range(wl.Hkv) if h_list is None else h_list
    K = torch.empty((len(bs), len(hs), n, wl.d), dtype=wl.torch_dtype, device=device)
    V = torch.empty_like(K)
    for bi, b in enumerate(bs):
        for hi, h in enumerate(hs):
            K[bi, hi] = to_storage(normal((n, wl.d), device, wl.seed, ROLE["k"],
                                          layer, b, h), wl.dtype)
            V[bi, hi] = to_storage(normal((n, wl.d), device, wl.seed, ROLE["v"],
                                          layer, b, h), wl.dtype)
    return K, V


def kv_rows_device(wl: Workload, device, n_rows: int, layer: int = 0):
    """Level-0 K and V [B, Hkv, n_rows, d] drawn N(0,1) by the device's own
    generator (seeded per workload, role and layer) and rounded to the
    storage dtype.  For the largest cases, where drawing on the host would
    take minutes: the values are reproducible on one kind of device, and the
    oracle reads the very tensors the kernels read."""
    K = torch.empty((wl.B, wl.Hkv, n_rows, wl.d), dtype=wl.torch_dtype, device=device)
    V = torch.empty_like(K)
    for X, role in ((K, "k"), (V, "v")):
        g = generator(device, wl.seed, ROLE[role], layer, "device")
        for b in range(wl.B):
            for h in range(wl.Hkv):
                X[b, h] = to_storage(torch.randn((n_rows, wl.d), generator=g, device=device,
                                                 dtype=torch.float32), wl.dtype)
    return K, V


def plant_needles(wl: Workload, K: torch.Tensor, q: torch.Tensor, layer: int = 0,
                  b_list=None, h_list=None):
    """Overwrite wl.n_needles rows per (sequence, KV head) of K with keys of
    norm sqrt(d) at cosine 0.9 to the unit mean of that head's decode queries.
    Returns the needle positions [len(b), len(h), n_needles] (int64, CPU)."""
    bs = range(wl.B) if b_list is None else b_list
    hs = range(wl.Hkv) if h_list is None else h_list
    pos_all = torch.zeros((len(bs), len(hs), wl.n_needles), dtype=torch.int64)
    if wl.n_needles == 0:
        return pos_all
    dev = K.device
    for bi, b in enumerate(bs):
        for hi, h in enumerate(hs):
            qg = q[b, :, h * wl.G:(h + 1) * wl.G].float().reshape(-1, wl.d)
            qh = qg.mean(0)
            qh = qh / qh.norm()
            u = normal((wl.n_needles, wl.d), dev, wl.seed, ROLE["needle"],
                       layer, b, h)
            u = u - (u @ qh)[:, None] * qh[None, :]
            u = u / u.norm(dim=1, keepdim=True)
            key = (wl.d ** 0.5) * (0.9 * qh[None, :] + (0.19 ** 0.5) * u)
            g = generator("cpu", wl.seed, ROLE["needle_pos"], layer, b, h)
            pos = torch.randint(0, K.shape[2], (wl.n_needles,), generator=g)
            K[bi, hi, pos.to(dev)] = to_storage(key, wl.dtype)
            pos_all[bi, hi] = pos
    return pos_all


def new_rows(wl: Workload, device, n: int, role: str, step: int = 0,
             layer: int = 0):
    """Fresh K, V, q rows for appended tokens: K,V [B, Hkv, n, d], q [B, n, Hq, d]."""
    k = normal((wl.B, wl.Hkv, n, wl.d), device, wl.seed, ROLE[role], layer, step, 0)
    v = normal((wl.B, wl.Hkv, n, wl.d), device, wl.seed, ROLE[role], layer, step, 1)
    q = normal((wl.B, n, wl.Hq, wl.d), device, wl.seed, ROLE[role], layer, step, 2)
    return (to_storage(k, wl.dtype), to_storage(v, wl.dtype),
            to_storage(q, wl.dtype))
