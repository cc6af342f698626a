"""RecSA hot-path benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 524k] [--no-cpu-baseline]

Workload (default "524k"): one Qwen3-4B-shaped attention layer (8 KV heads,
32 query heads, head dim 128, bf16, C=16, k=256) holding L=524288 tokens of
seeded synthetic K/V (N(0,1), 16 planted needle keys per KV head).  One step
is the whole hot path once:
  prefill: a 4096-query causal chunk at [L, L+4096) -- incremental tree
           build of the chunk's nodes, T-query selection, attention;
  decode : one token at t = L+4096 -- append, selection, attention, replayed
           as one HIP graph with a launch shape independent of L.
Inputs are resident in HBM before timing.  W untimed steps, then K timed
steps between two device synchronisations; HIP events on the stream the
kernels run on split each step into its prefill and decode parts.

Printed: one JSON line.  `value` is the decode latency per token in
microseconds (lower is better); prefill tokens/s, the full-tree build and
per-call splits ride along.  `roofline` is for the dominant decode kernel
measured in a separate instrumented pass; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload (rank 0, one thread).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROW_BYTES = 256                # one bf16 row of d=128


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def list_sizes(t, C, k, n_levels):
    """Data-free candidate-list sizes of the walk for a query at t (Eq. 3):
    returns {level: |A|} for levels n_levels-1 .. 0."""
    sizes = {}
    top = n_levels - 1
    n = (t >> (4 * top)) + 1
    sizes[top] = n
    for lvl in range(top - 1, -1, -1):
        kept = min(k, sizes[lvl + 1])
        sizes[lvl] = C * (kept - 1) + ((t >> (4 * lvl)) % C) + 1
    return sizes


def decode_rows(t, C, k, n_levels):
    """Rows one decode query must read per KV head: scored keys at every
    scored level, level-0 keys, and the value of every entry of E."""
    s = list_sizes(t, C, k, n_levels)
    scored = sum(s[lvl] - 1 for lvl in range(1, n_levels) if s[lvl] > k)
    summaries = sum(s[lvl] - k for lvl in range(1, n_levels) if s[lvl] > k)
    n_e = s[0] + summaries
    return dict(scored_keys=scored, level0_keys=s[0], entries=n_e,
                rows=scored + s[0] + n_e, sizes=s)


def build_bytes(L, Hkv, n_levels, tb=0):
    """Bytes a build over tokens [tb, L) must move per sequence: the rotated
    copy of each level-0 key row (read K, write Kr), and per node its 16
    children's K and V rows read plus its K, V and Kr rows written."""
    total = (L - tb) * Hkv * 2 * ROW_BYTES
    for lvl in range(1, n_levels):
        n = (L >> (4 * lvl)) - (tb >> (4 * lvl))
        total += n * Hkv * (2 * 16 + 3) * ROW_BYTES
    return total


class Work:
    """Device-resident state of one benchmark workload (see module doc)."""


def setup_workload(name="524k", dev="cuda", level0_host=False):
    """Build the inputs of a workload in HBM and return the step closures.

    Level-0 K/V of L tokens plus the prefill chunk's rows and the decode
    token's row, the tree (levels >= 1 still empty), pooler, queries,
    positions, selection buffers, workspaces and outputs."""
    import torch

    import synth
    from long_context_kv_amd import recsa as R

    R.lib()                                     # fail loudly without the library
    wl = synth.WORKLOADS[name]
    w = Work()
    w.R, w.wl = R, wl
    L, T, B, Hkv, Hq, d = wl.L, max(wl.prefill_T, 1), wl.B, wl.Hkv, wl.Hq, wl.d
    t_dec = L + wl.prefill_T
    L_cap = t_dec + 64
    w.L, w.T, w.t_dec = L, T, t_dec
    log(f"workload {wl.name}: B={B} Hkv={Hkv} Hq={Hq} d={d} {wl.dtype} L={L} T={wl.prefill_T}")
    t0 = time.time()
    K0, V0 = synth.kv_rows(wl, dev, n_rows=L_cap)
    w.q_dec = synth.decode_queries(wl, dev)                        # [B, 1, Hq, d]
    w.needles = synth.plant_needles(wl, K0[:, :, :L], w.q_dec)
    w.pdict = synth.pooler_params(d, d, dev, wl.seed)
    w.pool = R.Pooler.from_dict(w.pdict, dev)
    w.tree = R.Tree.allocate(B, Hkv, d, L_cap, k=wl.k, dtype=wl.dtype, device=dev,
                             level0=(K0, V0), theta=wl.theta, level0_host=level0_host)
    tree = w.tree
    if level0_host:
        del K0, V0                              # level 0 now lives in pinned host memory
        torch.cuda.empty_cache()
    ck, cv, w.q_pre = synth.new_rows(wl, dev, T, "chunk")
    tree.K[0][:, :, L:L + T] = ck
    tree.V[0][:, :, L:L + T] = cv
    w.k_new = tree.K[0][:, :, t_dec].to(dev, copy=True).contiguous()
    w.v_new = tree.V[0][:, :, t_dec].to(dev, copy=True).contiguous()
    w.pos_pre = torch.arange(L, L + T, device=dev).view(1, T).expand(B, T).contiguous()
    w.pos_dec = torch.full((B,), t_dec, dtype=torch.int64, device=dev)
    w.ws_pre = R.workspace(tree, Hq, B * T)
    w.ws_dec = R.workspace(tree, Hq, B)
    w.sel_pre, w.cnt_pre, _ = tree.selection_buffers(B * T)
    w.sel_dec, w.cnt_dec, _ = tree.selection_buffers(B)
    w.out_pre = torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev)
    w.out_dec = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)

    def prefill():
        R.recsa_build_tree(tree, w.pool, L, L + T)
        R.recsa_select(tree, w.q_pre, Hq, T, w.pos_pre, w.sel_pre, w.cnt_pre, None, w.ws_pre)
        R.recsa_attn_prefill(tree, w.q_pre, Hq, T, w.pos_pre, w.sel_pre, w.cnt_pre, w.out_pre,
                             w.ws_pre)

    def decode():
        R.recsa_decode(tree, w.pool, w.k_new, w.v_new, w.q_dec, Hq, w.pos_dec, w.sel_dec,
                       w.cnt_dec, w.out_dec, w.ws_dec)

    def decode_split():
        R.recsa_append_decode(tree, w.pool, w.k_new, w.v_new, w.pos_dec)
        R.recsa_select(tree, w.q_dec, Hq, 1, w.pos_dec.view(B, 1), w.sel_dec, w.cnt_dec, None,
                       w.ws_dec)
        R.recsa_attn_decode(tree, w.q_dec, Hq, w.pos_dec, w.sel_dec, w.cnt_dec, w.out_dec,
                            w.ws_dec)

    def build_full():
        R.recsa_build_tree(tree, w.pool, 0, L)

    w.prefill, w.decode, w.decode_split, w.build_full = prefill, decode, decode_split, build_full
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s; tree levels={tree.n_levels}")
    return w


def capture_decode(w, fn=None):
    """Capture a decode step as one HIP graph (its launch shape is fixed)."""
    import torch
    fn = fn or w.decode
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="524k")
    ap.add_argument("--decode-reps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="counter pass only: a 512 MiB device copy (the calibration kernel), "
                         "then the workload's fused decode step 5 times and one prefill "
                         "chunk; prints no result")
    ap.add_argument("--distill", action="store_true",
                    help="measure the pooler distillation losses (Eq. 6 over every position "
                         "of a 32768-token sequence, Eq. 7 over every node) instead")
    ap.add_argument("--offload", action="store_true",
                    help="measure decode and prefill with level 0 of the cache in pinned host "
                         "memory (read over PCIe in place) instead")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.pmc_pass:
        pmc_pass(args.workload)
        return
    if args.distill:
        bench_distill(args)
        return
    if args.offload:
        bench_offload(args)
        return
    w = setup_workload(args.workload)
    wl, tree, pool, R = w.wl, w.tree, w.pool, w.R
    L, T, B, Hkv, Hq, d = w.L, w.T, wl.B, wl.Hkv, wl.Hq, wl.d
    t_dec = w.t_dec
    prefill, decode = w.prefill, w.decode
    k_new, v_new, pos_dec, q_dec, q_pre = w.k_new, w.v_new, w.pos_dec, w.q_dec, w.q_pre
    pos_pre, ws_pre, ws_dec = w.pos_pre, w.ws_pre, w.ws_dec
    sel_pre, cnt_pre, sel_dec, cnt_dec = w.sel_pre, w.cnt_pre, w.sel_dec, w.cnt_dec
    out_pre, out_dec, pdict = w.out_pre, w.out_dec, w.pdict

    # ------------------------------------------------------ full tree build
    ev = lambda: torch.cuda.Event(enable_timing=True)
    build_ms = []
    for _ in range(3):
        a, b = ev(), ev()
        a.record()
        w.build_full()
        b.record()
        torch.cuda.synchronize()
        build_ms.append(a.elapsed_time(b))
    build_s = sorted(build_ms)[1] / 1e3
    bb = build_bytes(L, Hkv, tree.n_levels) * B
    log(f"full build over {L} tokens: {build_s * 1e3:.3f} ms, {bb / build_s / 1e9:.0f} GB/s")

    graph = capture_decode(w)

    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # one step = one prefill chunk, then one decode token (a single launch;
    # its graph replay is timed separately below)
    evs = [(ev(), ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for e0, e1, e2 in evs:
        e0.record()
        prefill()
        e1.record()
        decode()
        e2.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    pre_ms = [a.elapsed_time(b) for a, b, _ in evs]
    dec_ms = [b.elapsed_time(c) for _, b, c in evs]
    log(f"timed {args.steps} steps in {wall:.3f}s")

    # decode alone, many replays (latency distribution)
    reps = [(ev(), ev()) for _ in range(args.decode_reps)]
    for a, b in reps:
        a.record()
        graph.replay()
        b.record()
    torch.cuda.synchronize()
    dec_rep_us = sorted(a.elapsed_time(b) * 1e3 for a, b in reps)
    if torch.count_nonzero(R.decode_error_words(ws_dec, tree, Hq)).item() or \
            not torch.isfinite(out_dec).all():
        raise RuntimeError("a replayed decode step reported an error word or a non-finite output")

    # the same decode step as three calls (append, select, attention)
    graph_split = capture_decode(w, w.decode_split)
    reps2 = [(ev(), ev()) for _ in range(50)]
    for a, b in reps2:
        a.record()
        graph_split.replay()
        b.record()
    torch.cuda.synchronize()
    split_rep_us = sorted(a.elapsed_time(b) * 1e3 for a, b in reps2)
    # restore the fused step's outputs for anything read later
    graph.replay()
    torch.cuda.synchronize()

    # ------------------------------------------- instrumented per-call pass
    def timed(fn, n=20):
        xs = []
        for _ in range(n):
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            xs.append((a, b))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e3 for a, b in xs)
        return ts[len(ts) // 2]
    split = {
        "decode_fused_us": timed(lambda: R.recsa_decode(tree, pool, k_new, v_new, q_dec, Hq, pos_dec,
                                                        sel_dec, cnt_dec, out_dec, ws_dec)),
        "decode_append_us": timed(lambda: R.recsa_append_decode(tree, pool, k_new, v_new, pos_dec)),
        "decode_select_us": timed(lambda: R.recsa_select(tree, q_dec, Hq, 1, pos_dec.view(B, 1),
                                                         sel_dec, cnt_dec, None, ws_dec)),
        "decode_attn_us": timed(lambda: R.recsa_attn_decode(tree, q_dec, Hq, pos_dec, sel_dec,
                                                            cnt_dec, out_dec, ws_dec)),
        "prefill_build_us": timed(lambda: R.recsa_build_tree(tree, pool, L, L + T), 5),
        "prefill_select_us": timed(lambda: R.recsa_select(tree, q_pre, Hq, T, pos_pre, sel_pre,
                                                          cnt_pre, None, ws_pre), 5),
        "prefill_attn_us": timed(lambda: R.recsa_attn_prefill(tree, q_pre, Hq, T, pos_pre, sel_pre,
                                                              cnt_pre, out_pre, ws_pre), 5),
    }
    log("split " + json.dumps({k_: round(v, 1) for k_, v in split.items()}))

    # ------------------------------------------------------------- numbers
    dr = decode_rows(t_dec, 16, wl.k, tree.n_levels)
    dec_bytes = dr["rows"] * ROW_BYTES * Hkv * B
    dec_us = float(np.mean(dec_ms)) * 1e3
    pre_s = float(np.mean(pre_ms)) / 1e3
    fused_gbs = dec_bytes / (split["decode_fused_us"] * 1e-6) / 1e9
    traffic_b = measured_traffic(args.workload)
    roof = {
        "kernel": "decode_fused_kernel (recsa_decode: append + select + attention), "
                  "decode at t=%d" % t_dec,
        "bound": "hbm", "achieved": round(fused_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(fused_gbs / HBM_PEAK_GBS, 4),
        "traffic": (round(traffic_b / (split["decode_fused_us"] * 1e-6) / 1e9, 1)
                    if traffic_b else None),
        "traffic_bytes_per_launch": traffic_b,
        "algorithmic_bytes_per_launch": dec_bytes,
        "avg_launch_us": round(split["decode_fused_us"], 2),
    }
    step_gbs = dec_bytes / (dec_us * 1e-6) / 1e9
    # prefill scoring: 2 d flops per (query head, scored candidate); the
    # select call also files the candidates and runs the top-k, so the
    # fraction below is a lower bound for the scoring kernel itself
    g_q = Hq // Hkv
    scored = sum(decode_rows(t, 16, wl.k, tree.n_levels)["scored_keys"] for t in range(L, L + T))
    score_flops = scored * 2 * d * g_q * Hkv * B
    sel_tflops = score_flops / (split["prefill_select_us"] * 1e-6) / 1e12

    result = {
        "metric": "RecSA decode µs/token & prefill tok/s at 524K; % HBM / MFMA peak",
        "value": round(dec_us, 2),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: 1 layer, {Hkv} KV heads, {Hq} query heads, d={d}, "
                               f"{wl.dtype}, L={L}, C=16, k={wl.k}; decode B={B} at t={t_dec}; "
                               f"prefill chunk T={T} at [{L},{L + T})",
                   "seq_len": L, "global_batch": B, "prefill_T": T},
        "decode_us_per_token": round(dec_us, 2),
        "decode_us_median_replay": round(dec_rep_us[len(dec_rep_us) // 2], 2),
        "decode_us_p10_p90": [round(dec_rep_us[len(dec_rep_us) // 10], 2),
                              round(dec_rep_us[(9 * len(dec_rep_us)) // 10], 2)],
        "decode_split_calls_us_median": round(split_rep_us[len(split_rep_us) // 2], 2),
        "decode_algorithmic_MB": round(dec_bytes / 1e6, 2),
        "decode_step_GBs": round(step_gbs, 1),
        "decode_step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "prefill_tok_s": round(B * T / pre_s, 1),
        "prefill_ms_per_chunk": round(pre_s * 1e3, 3),
        "build_full_ms": round(build_s * 1e3, 3),
        "build_full_GBs": round(bb / build_s / 1e9, 1),
        "build_full_hbm_frac": round(bb / build_s / 1e9 / HBM_PEAK_GBS, 4),
        "split_us": {k_: round(v, 1) for k_, v in split.items()},
        "prefill_scoring": {"algorithmic_GFLOP": round(score_flops / 1e9, 1),
                            "select_TFLOPs": round(sel_tflops, 1), "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                            "select_frac": round(sel_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                            "dtype": "bf16 operands, fp32 accumulate (v_mfma_f32_16x16x32_bf16)"},
        "roofline": roof,
        "cache_state": "decode replays after a prefill chunk; levels >= 1 (~134 MB) fit the 256 MB MALL",
    }

    # ------------------------------------------------------- CPU baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, tree, pdict, q_dec, q_pre, t_dec, L, T)
    print(json.dumps(result), flush=True)


COPY_BYTES = 512 << 20
# sources of the fused decode kernel: a counter summary counts only while
# their hash matches the one recorded with it
FUSED_SOURCES = ("long_context_kv_amd/csrc/decode_fused.hip", "long_context_kv_amd/csrc/recsa_common.hpp",
                 "long_context_kv_amd/csrc/recsa_device.hpp", "long_context_kv_amd/csrc/recsa_mfma.hpp",
                 "long_context_kv_amd/csrc/recsa_pool.hpp", "long_context_kv_amd/csrc/recsa_kernels.hpp",
                 "include/recsa.h")


def fused_sources_sha():
    h = hashlib.sha256()
    for f in FUSED_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per fused-decode launch (FETCH_SIZE and WRITE_SIZE, each
    scaled by its reading of a plain copy of known size) from the committed
    counter summary of this workload; None if there is none or the kernel's
    sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"decode_fused_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        txt = fh.read()
    nb = re.search(r"traffic_bytes_per_launch:\s*(\d+)", txt)
    sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]+)", txt)
    if not (nb and sha) or sha.group(1) != fused_sources_sha():
        return None
    return int(nb.group(1))


def pmc_pass(name):
    """The launches a hardware-counter run reads: one plain device copy of
    COPY_BYTES (read once, written once), then the workload's fused decode
    step, five times, after the full build, then one prefill chunk."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    w = setup_workload(name)
    w.build_full()
    for _ in range(5):
        w.decode()
    w.prefill()
    torch.cuda.synchronize()
    log(f"pmc pass done: copy of {COPY_BYTES} bytes, 5 fused decode steps, one prefill chunk")


def cpu_baseline(wl, tree, pdict, q_dec, q_pre, t_dec, L, T):
    """The CPU oracle on one thread, on a bounded sample of the same workload:
    KV head 0 of sequence 0.  Timed: its tree build over t_dec+1 tokens, 8
    decode walks+softmaxes at t_dec (the 8 query-head groups against that
    head's tree) and 256 evenly spaced prefill queries of the chunk; each is
    scaled to all B*Hkv heads."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import recsa_oracle as O
    from tests import parity as PY

    heads = wl.Hkv * wl.B
    G = wl.Hq // wl.Hkv
    with threadpool_limits(limits=1):
        K0 = PY.to64(tree.K[0][0, 0, :t_dec + 1])
        V0 = PY.to64(tree.V[0][0, 0, :t_dec + 1])
        P = PY.oracle_pooler(pdict)
        t0 = time.time()
        Kt, Vt = O.build_tree(K0, V0, 16, tree.n_levels, P, wl.dtype)
        build_s = time.time() - t0
        cos, sin = O.rope_table(wl.d, 16 * wl.k, wl.theta)
        qd = PY.to64(q_dec[0, 0])                            # [Hq, d]
        t1 = time.time()
        for j in range(wl.Hkv):
            O.decode_reference(qd[j * G:(j + 1) * G], t_dec, Kt, Vt, 16, wl.k, cos, sin, wl.dtype)
        dec_s = (time.time() - t1) / wl.Hkv
        qp = PY.to64(q_pre[0, :, :G])
        idx = np.linspace(0, T - 1, 512).astype(int)
        t2 = time.time()
        for i in idx:
            t = L + int(i)
            Ktt = [Kt[0][: t + 1]] + [Kt[lv][: (t + 1) >> (4 * lv)] for lv in range(1, len(Kt))]
            Vtt = [Vt[0][: t + 1]] + [Vt[lv][: (t + 1) >> (4 * lv)] for lv in range(1, len(Vt))]
            O.decode_reference(qp[i], t, Ktt, Vtt, 16, wl.k, cos, sin, wl.dtype)
        pre_s = (time.time() - t2) / len(idx)
    total = time.time() - t0
    log(f"cpu baseline ({total:.1f}s): build/head {build_s:.2f}s, decode/head {dec_s:.3f}s, "
        f"prefill query/head {pre_s:.4f}s")
    return {
        "value": round(dec_s * heads * 1e6, 1), "unit": "us/token", "cores": 1, "kind": "oracle",
        "sample": (f"KV head 0 of {heads}, one thread: oracle tree build over {t_dec + 1} tokens, "
                   f"8 decode walks+softmaxes at t={t_dec} and 512 evenly spaced queries of the "
                   f"{T}-query prefill chunk, each scaled x{heads} heads ({total:.1f}s of CPU work)"),
        "prefill_tok_s": round(1.0 / (pre_s * heads), 3),
        "build_full_ms": round(build_s * heads * 1e3, 1),
    }


FP32_MFMA_PEAK_TFLOPS = 157.3
PCIE_PEAK_GBS = 63.0           # PCIe 5.0 x16, one direction, after 128b/130b encoding


def bench_offload(args):
    """The workload's decode step and prefill chunk with level 0 (K, V and
    the rotated keys Kr) in pinned host memory and levels >= 1 in HBM.  The
    kernels are the device-resident ones; each reads the level-0 rows it
    selected straight from host memory over PCIe.  Roofline: the level-0
    bytes one decode must read (Kr and V rows of A^(0) per KV head) against
    the PCIe peak."""
    import numpy as np
    import torch

    w = setup_workload(args.workload, level0_host=True)
    wl, tree, R = w.wl, w.tree, w.R
    L, T, B, Hkv, Hq, d = w.L, w.T, wl.B, wl.Hkv, wl.Hq, wl.d
    ev = lambda: torch.cuda.Event(enable_timing=True)
    a, b = ev(), ev()
    a.record()
    w.build_full()
    b.record()
    torch.cuda.synchronize()
    build_ms = a.elapsed_time(b)
    log(f"full build with level 0 in host memory: {build_ms:.1f} ms")
    for _ in range(args.warmup):
        w.prefill()
    torch.cuda.synchronize()
    pre = []
    for _ in range(args.steps):
        a, b = ev(), ev()
        a.record()
        w.prefill()
        b.record()
        pre.append((a, b))
    torch.cuda.synchronize()
    pre_ms = sorted(x.elapsed_time(y) for x, y in pre)[len(pre) // 2]
    graph = capture_decode(w)
    for _ in range(5):
        graph.replay()
    reps = [(ev(), ev()) for _ in range(args.decode_reps)]
    for x, y in reps:
        x.record()
        graph.replay()
        y.record()
    torch.cuda.synchronize()
    dec = sorted(x.elapsed_time(y) * 1e3 for x, y in reps)
    dec_us = dec[len(dec) // 2]
    err = torch.count_nonzero(R.decode_error_words(w.ws_dec, tree, Hq)).item()
    if err:
        raise RuntimeError("fused decode reported a timed-out wait")
    sizes = list_sizes(w.t_dec, 16, wl.k, tree.n_levels)
    host_bytes = 2 * sizes[0] * ROW_BYTES * Hkv * B
    gbs = host_bytes / (dec_us * 1e-6) / 1e9
    result = {
        "metric": "RecSA decode µs/token with level 0 in host memory (KV offload); "
                  "% of PCIe peak",
        "value": round(dec_us, 2), "unit": "us/token", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(pre_ms + dec_us / 1e3, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name} with level 0 (K, V, Kr) in pinned host memory: "
                               f"1 layer, {Hkv} KV heads, {Hq} query heads, d={d}, {wl.dtype}, "
                               f"L={L}, C=16, k={wl.k}; decode B={B} at t={w.t_dec}; "
                               f"prefill chunk T={wl.prefill_T}",
                   "seq_len": L, "global_batch": B},
        "decode_us_p10_p90": [round(dec[len(dec) // 10], 2), round(dec[(9 * len(dec)) // 10], 2)],
        "prefill_ms_per_chunk": round(pre_ms, 3),
        "prefill_tok_s": round(B * T / (pre_ms * 1e-3), 1),
        "build_full_ms": round(build_ms, 1),
        "gpu_resident_bytes": int(sum(x.numel() * x.element_size()
                                      for name in ("K", "V", "Kr")
                                      for x in getattr(tree, name)[1:])),
        "host_resident_bytes": int(3 * tree.K[0].numel() * tree.K[0].element_size()),
        "roofline": {"kernel": "decode_fused_kernel, level-0 reads over PCIe",
                     "bound": "pcie", "achieved": round(gbs, 2), "peak": PCIE_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / PCIE_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_host_bytes_per_launch": host_bytes},
    }
    print(json.dumps(result), flush=True)


def bench_distill(args):
    """Eq. 6 and Eq. 7 on the distillation workload: one step = selection
    with importances for every position of the sequence, the KL terms of
    every (query, KV head, scored level) with the teacher distributions, the
    shift penalty of every level, the KL's gradient with respect to every
    node key, and the pooler backward of every level from that gradient plus
    the penalty.  Roofline: the teacher's dense logits, 2 d flops per (query head,
    key) pair with key <= query, executed as three bf16 matrix products per
    pair (split operands); the whole recsa_distill_kl call is charged, so the
    fraction is a lower bound."""
    import numpy as np
    import torch

    import synth
    from long_context_kv_amd import recsa as R

    R.lib()
    wl = synth.WORKLOADS["distill_32k"]
    L, B, Hkv, Hq, d, dev = wl.L, wl.B, wl.Hkv, wl.Hq, wl.d, "cuda"
    T = L
    log(f"workload {wl.name}: B={B} Hkv={Hkv} Hq={Hq} d={d} {wl.dtype} L={L} k={wl.k}, "
        f"{T} queries per sequence")
    K0, V0 = synth.kv_rows(wl, dev, n_rows=L)
    pdict = synth.pooler_params(d, d, dev, wl.seed)
    pool = R.Pooler.from_dict(pdict, dev)
    tree = R.Tree.allocate(B, Hkv, d, L, k=wl.k, dtype=wl.dtype, device=dev, level0=(K0, V0),
                           theta=wl.theta)
    R.recsa_build_tree(tree, pool, 0, L)
    q = synth.to_storage(synth.normal((B, T, Hq, d), dev, wl.seed, ROLE_DISTILL_Q), wl.dtype)
    pos = torch.arange(T, device=dev).view(1, T).expand(B, T).contiguous()
    ws = R.workspace(tree, Hq, B * T)
    sel, cnt, imp = tree.selection_buffers(B * T, with_importance=True)
    dws = torch.empty(R.recsa_distill_workspace_bytes(tree, Hq, B * T), dtype=torch.uint8,
                      device=dev)
    kl = torch.empty((B, T, Hkv, tree.n_sel), dtype=torch.float32, device=dev)
    sws = torch.empty(R.recsa_shift_workspace_bytes(tree), dtype=torch.uint8, device=dev)
    pen = torch.empty((tree.n_levels - 1, d + 2), dtype=torch.float32, device=dev)

    def select():
        R.recsa_select(tree, q, Hq, T, pos, sel, cnt, imp, ws)

    def distill():
        R.recsa_distill_kl(tree, q, Hq, T, pos, sel, cnt, imp, wl.theta, kl, dws,
                           teacher=teacher)

    def shift():
        R.recsa_shift_penalty(tree, pool, L, pen, sws)

    # the KL's gradient with respect to every node key, then the pooler
    # backward of every level from it plus the shift penalty with weight 1
    levels = range(1, tree.n_levels)
    teacher = torch.empty((B * T, Hkv, tree.n_sel, 16 * wl.k), dtype=torch.float32, device=dev)
    kws = torch.empty(R.recsa_distill_key_grad_workspace_bytes(tree, Hq, B * T),
                      dtype=torch.uint8, device=dev)
    kbuf, dKs = R.key_grad_buffer(tree)
    bws = {lv: torch.empty(R.recsa_pooler_backward_workspace_bytes(tree, pool, lv),
                           dtype=torch.uint8, device=dev) for lv in levels}
    grads = {lv: R.pooler_grad_buffers(pool) for lv in levels}

    def key_grad():
        R.recsa_distill_key_grad(tree, q, Hq, T, pos, sel, cnt, imp, teacher, ws, kbuf, kws)

    def backward():
        for lv in levels:
            R.recsa_pooler_backward(tree, pool, lv, L, dKs[lv - 1], pen[lv - 1], 1.0, grads[lv],
                                    bws[lv])

    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        select(); distill(); shift(); key_grad(); backward()
    torch.cuda.synchronize()
    evs = [tuple(ev() for _ in range(6)) for _ in range(args.steps)]
    w0 = time.perf_counter()
    for e0, e1, e2, e3, e4, e5 in evs:
        e0.record(); select(); e1.record(); distill(); e2.record(); shift(); e3.record()
        key_grad(); e4.record(); backward(); e5.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    med = lambda xs: sorted(xs)[len(xs) // 2]
    sel_ms = med([x[0].elapsed_time(x[1]) for x in evs])
    kl_ms = med([x[1].elapsed_time(x[2]) for x in evs])
    sh_ms = med([x[2].elapsed_time(x[3]) for x in evs])
    kg_ms = med([x[3].elapsed_time(x[4]) for x in evs])
    bw_ms = med([x[4].elapsed_time(x[5]) for x in evs])
    step_ms = med([x[0].elapsed_time(x[5]) for x in evs])
    pairs = sum(int(t) + 1 for t in range(T)) * B          # (query, key <= query) pairs
    flops = 2.0 * d * Hq * pairs
    tflops = flops / (kl_ms * 1e-3) / 1e12
    klv = kl.cpu().numpy()
    result = {
        "metric": "RecSA pooler distillation step (Eq. 6 over every position + Eq. 7, the KL's "
                  "key gradient and the pooler backward of every level) at the 32K training "
                  "length; ms per layer",
        "value": round(step_ms, 3), "unit": "ms/layer-step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: 1 layer, {Hkv} KV heads, {Hq} query heads, d={d}, "
                               f"{wl.dtype}, L={L}, C=16, k={wl.k}; every position a query",
                   "seq_len": L, "global_batch": B},
        "split_ms": {"select_with_importance": round(sel_ms, 3), "distill_kl": round(kl_ms, 3),
                     "shift_penalty": round(sh_ms, 3), "kl_key_grad": round(kg_ms, 3),
                     "pooler_backward_all_levels": round(bw_ms, 3)},
        "queries_per_s": round(B * T / (step_ms * 1e-3), 1),
        "roofline": {"kernel": "recsa_distill_kl (absolute RoPE table + teacher_lse_kernel + "
                               "distill_kl_kernel), charged whole",
                     "bound": "mfma", "achieved": round(3 * tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(3 * tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_TFLOP_per_launch": round(flops / 1e12, 3),
                     "executed_bf16_TFLOP_per_launch": round(3 * flops / 1e12, 3),
                     "fp32_equivalent_TFLOPs": round(tflops, 2),
                     "fp32_equivalent_frac_of_fp32_peak": round(tflops / FP32_MFMA_PEAK_TFLOPS, 4),
                     "dtype": "bf16 x3 split (hi.hi + hi.lo + lo.hi per product, "
                              "v_mfma_f32_16x16x32_bf16, float32 accumulate)"},
        "kl_mean_per_level": [round(float(x), 5) for x in klv.reshape(-1, tree.n_sel).mean(0)],
        "shift_penalty_per_level": [round(float(x), 6) for x in pen[:, d + 1].cpu().numpy()],
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_distill(wl, tree, pdict, q, L)
    print(json.dumps(result), flush=True)


ROLE_DISTILL_Q = 11


def cpu_baseline_distill(wl, tree, pdict, q, L):
    """The oracle on one thread: KV head 0, 400 evenly spaced positions of the
    sequence (walk + Eq. 6 each), scaled to every position and KV head."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import recsa_oracle as O
    from tests import parity as PY

    G = wl.Hq // wl.Hkv
    with threadpool_limits(limits=1):
        K0 = PY.to64(tree.K[0][0, 0, :L])
        V0 = PY.to64(tree.V[0][0, 0, :L])
        P = PY.oracle_pooler(pdict)
        t0 = time.time()
        Kt, _ = O.build_tree(K0, V0, 16, tree.n_levels, P, wl.dtype)
        cos, sin = O.rope_table(wl.d, 16 * wl.k, wl.theta)
        qn = PY.to64(q[0, :, :G])
        idx = np.linspace(0, L - 1, 400).astype(int)
        t1 = time.time()
        for t in idx:
            t = int(t)
            D = O.n_levels_for(t, 16, wl.k)
            Ktt = ([Kt[0][: t + 1]] + [Kt[lv][: (t + 1) >> (4 * lv)]
                                       for lv in range(1, len(Kt))])[: max(D, 1)]
            tr = O.walk(qn[t], t, Ktt, 16, wl.k, cos, sin, wl.dtype)
            O.distill_kl(qn[t], t, tr, K0[: t + 1], 16, wl.theta)
        per_q = (time.time() - t1) / len(idx)
    total = time.time() - t0
    heads = wl.Hkv * wl.B
    scaled_ms = per_q * L * heads * 1e3
    log(f"cpu baseline distill ({total:.1f}s): {per_q * 1e3:.1f} ms per (query, head)")
    return {"value": round(scaled_ms, 1), "unit": "ms/layer-step", "cores": 1, "kind": "oracle",
            "sample": (f"KV head 0 of {heads}, one thread: oracle walk + Eq. 6 at 400 evenly "
                       f"spaced positions of {L}, scaled x{L} positions x{heads} heads "
                       f"({total:.1f}s of CPU work; Eq. 7, the key gradient and the pooler backward not included)")}


if __name__ == "__main__":
    main()
