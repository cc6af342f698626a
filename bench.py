"""RecSA hot-path benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 524k] [--no-cpu-baseline]
                    [--no-config5]

Workload (default "524k"): one Qwen3-4B-shaped attention layer (8 KV heads,
32 query heads, head dim 128, bf16, C=16, k=256) holding L=524288 tokens of
seeded synthetic K/V (N(0,1), 16 planted needle keys per KV head).  One step
is the whole hot path once:
  prefill: a 4096-query causal chunk at [L, L+4096) -- incremental tree
           build of the chunk's nodes, T-query selection, attention;
  decode : one new token at t = L+4096+s (step s) with its own fresh q, k, v
           -- append, selection, attention in one launch whose shape does not
           depend on L.
Inputs are resident in HBM before timing.  W untimed steps, then K timed
steps between two device synchronisations; HIP events on the stream the
kernels run on split each step into its prefill and decode parts.  Then the
decode alone: >= 200 consecutive tokens, each with fresh inputs and captured
as its own HIP graph, replayed back to back (warm caches) and again each
after a 512 MB buffer is rewritten (last-level cache scrubbed), and the same
tokens as direct launches (warm); medians.  `roofline` averages the fused
decode launches of the timed steps.

The 4-layer 2M-token configuration (full build of each layer, an 8192-query
prefill chunk per layer, then 256 decode steps over the 4 layers with fresh
inputs) runs after the headline unless --no-config5.

Printed: one JSON line.  `value` is the decode latency per token in
microseconds (lower is better) in the timed steps; prefill tokens/s, the
full-tree build, per-call splits and the other configuration ride along.
`roofline` is for the dominant decode kernel; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload on the host's cores.
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
    """Algorithmic bytes of a build over tokens [tb, L) per sequence: per
    complete node, its 16 children's K and V rows read and its own K and V
    rows written, (2C + 2) rows."""
    total = 0
    for lvl in range(1, n_levels):
        n = (L >> (4 * lvl)) - (tb >> (4 * lvl))
        total += n * Hkv * (2 * 16 + 2) * ROW_BYTES
    return total


def build_bytes_with_rotated_keys(L, Hkv, n_levels, tb=0):
    """What this build also moves for its rotated-key copy Kr: each level-0
    key row read and its rotated row written, one Kr row per node."""
    total = build_bytes(L, Hkv, n_levels, tb) + (L - tb) * Hkv * 2 * ROW_BYTES
    for lvl in range(1, n_levels):
        total += ((L >> (4 * lvl)) - (tb >> (4 * lvl))) * Hkv * ROW_BYTES
    return total


def prefill_attention_work(L, T, C, k, n_levels, G, Hkv, d):
    """Algorithmic work of the attention of a causal chunk at [L, L+T): flops
    2 d G (|A^(0)| + |E|) per (query, KV head) (level-0 logits and P V), and
    the unique bytes every query of an i.i.d. chunk touches -- in effect all
    of level 0's K and V rows plus the V rows of levels >= 1."""
    flops = 0
    for t in range(L, L + T):
        dr = decode_rows(t, C, k, n_levels)
        flops += 2 * d * G * (dr["level0_keys"] + dr["entries"]) * Hkv
    t_end = L + T
    uniq = 2 * t_end * Hkv * ROW_BYTES
    for lvl in range(1, n_levels):
        uniq += (t_end >> (4 * lvl)) * Hkv * ROW_BYTES
    return flops, uniq


class Work:
    """Device-resident state of one benchmark workload (see module doc)."""


def setup_workload(name="524k", dev="cuda", level0_host=False, n_decode=1, rotated_keys=True):
    """Build the inputs of a workload in HBM and return the step closures.

    Level-0 K/V of L tokens plus the prefill chunk's rows and the rows of
    n_decode decode tokens, the tree (levels >= 1 still empty), pooler,
    queries, positions, selection buffers, workspaces and outputs.  Decode
    slot i is token t_dec + i with its own query and K/V row (slot 0's query
    is the one the needles are planted for)."""
    import torch

    import synth
    from long_context_kv_amd import recsa as R

    R.lib()                                     # fail loudly without the library
    wl = synth.WORKLOADS[name]
    w = Work()
    w.R, w.wl = R, wl
    L, T, B, Hkv, Hq, d = wl.L, max(wl.prefill_T, 1), wl.B, wl.Hkv, wl.Hq, wl.d
    t_dec = L + wl.prefill_T
    L_cap = t_dec + n_decode + 64
    w.L, w.T, w.t_dec = L, T, t_dec
    log(f"workload {wl.name}: B={B} Hkv={Hkv} Hq={Hq} d={d} {wl.dtype} L={L} T={wl.prefill_T}")
    t0 = time.time()
    K0, V0 = synth.kv_rows(wl, dev, n_rows=L_cap)
    w.q_dec = synth.decode_queries(wl, dev)                        # [B, 1, Hq, d]
    w.needles = synth.plant_needles(wl, K0[:, :, :L], w.q_dec)
    w.pdict = synth.pooler_params(d, d, dev, wl.seed)
    w.pool = R.Pooler.from_dict(w.pdict, dev)
    w.tree = R.Tree.allocate(B, Hkv, d, L_cap, k=wl.k, dtype=wl.dtype, device=dev,
                             level0=(K0, V0), theta=wl.theta, level0_host=level0_host,
                             rotated_keys=rotated_keys)
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
    # decode slots: (q, k_new, v_new, pos) of token t_dec + i
    w.dec_in = [(w.q_dec, w.k_new, w.v_new, w.pos_dec)]
    for i in range(1, n_decode):
        w.dec_in.append((synth.decode_queries(wl, dev, step=i),
                         tree.K[0][:, :, t_dec + i].to(dev, copy=True).contiguous(),
                         tree.V[0][:, :, t_dec + i].to(dev, copy=True).contiguous(),
                         torch.full((B,), t_dec + i, dtype=torch.int64, device=dev)))
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

    def decode(i=0):
        q, kn, vn, pos = w.dec_in[i]
        R.recsa_decode(tree, w.pool, kn, vn, q, Hq, pos, w.sel_dec, w.cnt_dec, w.out_dec,
                       w.ws_dec)

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
    fn = fn or (lambda: w.decode(0))
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
    ap.add_argument("--no-rotated-keys", action="store_true",
                    help="keep no rotated-key copy Kr (K/V-only tree, 1/15 overhead): the "
                         "kernels rotate the key rows they read")
    ap.add_argument("--no-config5", action="store_true",
                    help="skip the 4-layer 2M-token configuration after the headline")
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
    n_dec = max(args.decode_reps, args.warmup + args.steps)
    w = setup_workload(args.workload, n_decode=n_dec, rotated_keys=not args.no_rotated_keys)
    wl, tree, pool, R = w.wl, w.tree, w.pool, w.R
    L, T, B, Hkv, Hq, d = w.L, w.T, wl.B, wl.Hkv, wl.Hq, wl.d
    t_dec = w.t_dec
    prefill, decode = w.prefill, w.decode
    k_new, v_new, pos_dec, q_dec, q_pre = w.k_new, w.v_new, w.pos_dec, w.q_dec, w.q_pre
    pos_pre, ws_pre, ws_dec = w.pos_pre, w.ws_pre, w.ws_dec
    sel_pre, cnt_pre, sel_dec, cnt_dec = w.sel_pre, w.cnt_pre, w.sel_dec, w.cnt_dec
    out_pre, out_dec, pdict = w.out_pre, w.out_dec, w.pdict
    ev = lambda: torch.cuda.Event(enable_timing=True)
    med = lambda xs: sorted(xs)[len(xs) // 2]

    # ------------------------------------------------------ full tree build
    build_ms = []
    for _ in range(5):
        a, b = ev(), ev()
        a.record()
        w.build_full()
        b.record()
        torch.cuda.synchronize()
        build_ms.append(a.elapsed_time(b))
    build_s = med(build_ms) / 1e3
    bb = build_bytes(L, Hkv, tree.n_levels) * B
    bb_kr = build_bytes_with_rotated_keys(L, Hkv, tree.n_levels) * B
    log(f"full build over {L} tokens: {build_s * 1e3:.3f} ms, {bb / build_s / 1e9:.0f} GB/s "
        f"algorithmic")

    # one step = one prefill chunk, then one new decode token (fresh q, k, v;
    # slot s is token t_dec + s, so the steps form a decode sequence)
    for s_ in range(args.warmup):
        prefill()
        decode(s_)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    evs = [(ev(), ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i, (e0, e1, e2) in enumerate(evs):
        e0.record()
        prefill()
        e1.record()
        decode(args.warmup + i)
        e2.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    pre_ms = [a.elapsed_time(b) for a, b, _ in evs]
    dec_ms = [b.elapsed_time(c) for _, b, c in evs]
    log(f"timed {args.steps} steps in {wall:.3f}s")

    # decode alone: each token its own graph (fresh inputs, t_dec + i), the
    # tokens replayed in order, warm, then each after a cache scrub
    graphs = [capture_decode(w, (lambda i=i: decode(i))) for i in range(n_dec)]

    def replay_all(scrub=None):
        xs = []
        for g in graphs:
            if scrub is not None:
                scrub.add_(1.0)
            a, b = ev(), ev()
            a.record()
            g.replay()
            b.record()
            xs.append((a, b))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in xs]
    first_us = replay_all()                            # every token appended once more
    warm_us = replay_all()

    def direct_all():
        xs = []
        for i in range(n_dec):
            a, b = ev(), ev()
            a.record()
            decode(i)
            b.record()
            xs.append((a, b))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in xs]
    direct_all()
    direct_us = direct_all()                           # the same tokens as direct launches
    scrub = torch.zeros(SCRUB_BYTES // 4, dtype=torch.float32, device="cuda")
    cold_us = replay_all(scrub)
    del scrub
    if torch.count_nonzero(R.decode_error_words(ws_dec, tree, Hq)).item() or \
            not torch.isfinite(out_dec).all():
        raise RuntimeError("a replayed decode step reported an error word or a non-finite output")
    graphs[0].replay()                                 # slot 0's outputs for what follows
    torch.cuda.synchronize()
    needle_recall = needle_recall_in_level0(w)

    # the same decode step as three calls (append, select, attention)
    graph_split = capture_decode(w, w.decode_split)
    reps2 = [(ev(), ev()) for _ in range(50)]
    for a, b in reps2:
        a.record()
        graph_split.replay()
        b.record()
    torch.cuda.synchronize()
    split_rep_us = sorted(a.elapsed_time(b) * 1e3 for a, b in reps2)
    graphs[0].replay()
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
        return med([a.elapsed_time(b) * 1e3 for a, b in xs])
    split = {
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
    graphs[0].replay()
    torch.cuda.synchronize()
    log("split " + json.dumps({k_: round(v, 1) for k_, v in split.items()}))

    # ------------------------------------------------------------- numbers
    dec_bytes_i = [decode_rows(t_dec + i, 16, wl.k, tree.n_levels)["rows"] * ROW_BYTES * Hkv * B
                   for i in range(n_dec)]
    dec_bytes = dec_bytes_i[0]
    dec_bytes_mean = float(np.mean(dec_bytes_i))
    dec_ms_us = [x * 1e3 for x in dec_ms]
    dec_us = med(dec_ms) * 1e3
    pre_s = med(pre_ms) / 1e3
    # the fused launches of the timed steps (each right after a prefill chunk)
    avg_us = float(np.mean(dec_ms_us))
    fused_gbs = dec_bytes_mean / (avg_us * 1e-6) / 1e9
    traffic_b = measured_traffic(args.workload)
    roof = {
        "kernel": "decode_fused_kernel (recsa_decode: append + select + attention), "
                  "mean of its %d event-timed launches in the timed steps: tokens from t=%d "
                  "with fresh q/k/v, each right after a prefill chunk" % (len(dec_ms_us), t_dec),
        "bound": "hbm", "achieved": round(fused_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(fused_gbs / HBM_PEAK_GBS, 4),
        "traffic": (round(traffic_b / (avg_us * 1e-6) / 1e9, 1) if traffic_b else None),
        "traffic_bytes_per_launch": traffic_b,
        "algorithmic_bytes_per_launch": round(dec_bytes_mean),
        "avg_launch_us": round(avg_us, 2),
    }
    step_gbs = dec_bytes / (dec_us * 1e-6) / 1e9
    # prefill scoring: 2 d flops per (query head, scored candidate); the
    # select call also files the candidates and runs the top-k, so the
    # fraction below is a lower bound for the scoring kernel itself
    g_q = Hq // Hkv
    scored = sum(decode_rows(t, 16, wl.k, tree.n_levels)["scored_keys"] for t in range(L, L + T))
    score_flops = scored * 2 * d * g_q * Hkv * B
    sel_tflops = score_flops / (split["prefill_select_us"] * 1e-6) / 1e12
    att_flops, att_uniq = prefill_attention_work(L, T, 16, wl.k, tree.n_levels, g_q, Hkv, d)
    att_flops *= B
    att_uniq *= B
    att_s = split["prefill_attn_us"] * 1e-6

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
                               f"{wl.dtype}, L={L}, C=16, k={wl.k}"
                               f"{'' if tree.Kr[0].numel() else ', no rotated-key copy'}; "
                               f"per step a prefill chunk "
                               f"T={T} at [{L},{L + T}) then decode B={B} of a new token from "
                               f"t={t_dec} with fresh q/k/v",
                   "seq_len": L, "global_batch": B, "prefill_T": T},
        "decode_us_per_token": round(dec_us, 2),
        "decode_note": "value: median over the timed steps of the decode token right after "
                       "each prefill chunk (the chunk's gathers leave the caches cold)",
        "decode_fresh_inputs_us_median_warm": round(med(warm_us), 2),
        "decode_fresh_inputs_us_median_scrubbed": round(med(cold_us), 2),
        "decode_fresh_inputs_us_median_warm_direct": round(med(direct_us), 2),
        "decode_fresh_note": "warm and scrubbed: each token its own HIP graph (torch.cuda.CUDAGraph "
                             "replay); warm_direct: the same tokens as direct launches",
        "decode_fresh_inputs_us_p10_p90_warm": [round(sorted(warm_us)[len(warm_us) // 10], 2),
                                                round(sorted(warm_us)[9 * len(warm_us) // 10], 2)],
        "decode_fresh_inputs_steps": n_dec,
        "decode_scrub": f"{SCRUB_BYTES >> 20} MB buffer rewritten before each scrubbed step "
                        "(MI355X last-level cache: 256 MB)",
        "decode_split_calls_us_median": round(split_rep_us[len(split_rep_us) // 2], 2),
        "decode_algorithmic_MB": round(dec_bytes / 1e6, 2),
        "decode_step_GBs": round(step_gbs, 1),
        "decode_step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "decode_hbm_frac_warm": round(dec_bytes_mean / (med(warm_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_hbm_frac_scrubbed": round(dec_bytes_mean / (med(cold_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "needle_recall_level0": needle_recall,
        "prefill_tok_s": round(B * T / pre_s, 1),
        "prefill_ms_per_chunk": round(pre_s * 1e3, 3),
        "build_full_ms": round(build_s * 1e3, 3),
        "build_full_GBs": round(bb / build_s / 1e9, 1),
        "build_full_hbm_frac": round(bb / build_s / 1e9 / HBM_PEAK_GBS, 4),
        "build_algorithmic_GB": round(bb / 1e9, 3),
        "build_with_rotated_keys_GB": round(bb_kr / 1e9, 3),
        "split_us": {k_: round(v, 1) for k_, v in split.items()},
        "prefill_scoring": {"algorithmic_GFLOP": round(score_flops / 1e9, 1),
                            "select_TFLOPs": round(sel_tflops, 1), "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                            "select_frac": round(sel_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                            "dtype": "bf16 operands, fp32 accumulate (v_mfma_f32_16x16x32_bf16)"},
        "prefill_attention": {"algorithmic_GFLOP": round(att_flops / 1e9, 1),
                              "unique_GB": round(att_uniq / 1e9, 3),
                              "ms": round(att_s * 1e3, 3),
                              "TFLOPs": round(att_flops / att_s / 1e12, 2),
                              "mfma_frac": round(att_flops / att_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                              "unique_GBs": round(att_uniq / att_s / 1e9, 1),
                              "unique_hbm_frac": round(att_uniq / att_s / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": roof,
    }

    # measured peaks of this device, for fractions beside the datasheet's
    mp = measured_peaks()
    result["measured_peaks"] = mp
    result["fractions_of_measured_peaks"] = {
        "decode_fused_of_copy": round(fused_gbs / mp["copy_GBs"], 4),
        "build_of_copy": round(bb / build_s / 1e9 / mp["copy_GBs"], 4),
        "prefill_scoring_of_gemm": round(sel_tflops / mp["bf16_gemm_TFLOPs"], 4),
        "prefill_attention_of_gemm": round(att_flops / att_s / 1e12 / mp["bf16_gemm_TFLOPs"], 4),
    }

    # ------------------------------------------------------- CPU baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, tree, pdict, q_dec, q_pre, t_dec, L, T,
                                              sel_dec.view(B, Hkv, tree.n_sel, tree.k))
    del graphs, graph_split, w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_config5 and args.workload == "524k":
        result["config5_2m_4layers"] = bench_config5(args)
    print(json.dumps(result), flush=True)


class Config5:
    """The 4-layer 2M-token configuration: 4 independent layers (own K/V,
    needles and pooler each), all resident in HBM at once.  Per layer: a full
    build over L tokens, then a causal prefill chunk of T queries at [L, L+T)
    (incremental build, selection, attention); then `steps` decode steps,
    each one new token per layer with fresh q, k, v (token L+T+s, layer after
    layer).  The prefill workspace is shared by the layers (they run one after
    another), and so is the decode workspace."""

    def __init__(self, dev="cuda", steps=None, layers=None):
        import torch

        import synth
        from long_context_kv_amd import recsa as R
        R.lib()
        wl = synth.WORKLOADS["2m_l4"]
        self.R, self.wl = R, wl
        self.L, self.T = wl.L, wl.prefill_T
        self.steps = wl.decode_steps if steps is None else steps
        self.n_layers = wl.n_layers if layers is None else layers
        self.t_dec = self.L + self.T
        L_cap = self.t_dec + self.steps + 64
        B, Hkv, Hq, d = wl.B, wl.Hkv, wl.Hq, wl.d
        self.layers = []
        for ly in range(self.n_layers):
            K0, V0 = synth.kv_rows_device(wl, dev, L_cap, layer=ly)
            q_dec = synth.decode_queries(wl, dev, layer=ly)
            needles = synth.plant_needles(wl, K0[:, :, :self.L], q_dec, layer=ly)
            pdict = synth.pooler_params(d, d, dev, wl.seed, layer=ly)
            tree = R.Tree.allocate(B, Hkv, d, L_cap, k=wl.k, dtype=wl.dtype, device=dev,
                                   level0=(K0, V0), theta=wl.theta)
            del K0, V0
            q_pre = synth.new_rows(wl, dev, self.T, "chunk", layer=ly)[2]
            dec = []
            for s_ in range(self.steps):
                q = q_dec if s_ == 0 else synth.decode_queries(wl, dev, step=s_, layer=ly)
                t = self.t_dec + s_
                dec.append((q, tree.K[0][:, :, t].clone().contiguous(),
                            tree.V[0][:, :, t].clone().contiguous(),
                            torch.full((B,), t, dtype=torch.int64, device=dev)))
            self.layers.append(dict(tree=tree, pool=R.Pooler.from_dict(pdict, dev), pdict=pdict,
                                    q_pre=q_pre, dec=dec, needles=needles))
        self.pos_pre = torch.arange(self.L, self.L + self.T, device=dev).view(1, self.T) \
            .expand(B, self.T).contiguous()
        t0 = self.layers[0]["tree"]
        self.ws_pre = R.workspace(t0, Hq, B * self.T)
        self.sel_pre, self.cnt_pre, _ = t0.selection_buffers(B * self.T)
        self.out_pre = torch.empty((B, self.T, Hq, d), dtype=torch.float32, device=dev)
        self.ws_dec = R.workspace(t0, Hq, B)
        self.sel_dec = [ly["tree"].selection_buffers(B)[:2] for ly in self.layers]
        self.out_dec = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
                        for _ in self.layers]
        torch.cuda.synchronize()

    def build(self, ly):
        x = self.layers[ly]
        self.R.recsa_build_tree(x["tree"], x["pool"], 0, self.L)

    def prefill(self, ly):
        R, x, Hq, T = self.R, self.layers[ly], self.wl.Hq, self.T
        R.recsa_build_tree(x["tree"], x["pool"], self.L, self.L + T)
        R.recsa_select(x["tree"], x["q_pre"], Hq, T, self.pos_pre, self.sel_pre, self.cnt_pre,
                       None, self.ws_pre)
        R.recsa_attn_prefill(x["tree"], x["q_pre"], Hq, T, self.pos_pre, self.sel_pre,
                             self.cnt_pre, self.out_pre, self.ws_pre)

    def decode(self, s_):
        R, Hq = self.R, self.wl.Hq
        for ly, x in enumerate(self.layers):
            q, kn, vn, pos = x["dec"][s_]
            sel, cnt = self.sel_dec[ly]
            R.recsa_decode(x["tree"], x["pool"], kn, vn, q, Hq, pos, sel, cnt, self.out_dec[ly],
                           self.ws_dec)


def bench_config5(args):
    """Measure the 4-layer 2M-token configuration (class Config5): the full
    build of every layer, the prefill chunk of every layer, and 256 decode
    steps of the 4 layers; rooflines by the algorithmic bytes of the build
    and of each decode step."""
    import numpy as np
    import torch
    log("config 5: 4 layers x 2M tokens")
    t0 = time.time()
    c = Config5()
    wl, R = c.wl, c.R
    tree0 = c.layers[0]["tree"]
    n_lv, Hkv, B, T = tree0.n_levels, wl.Hkv, wl.B, c.T
    log(f"config 5 inputs ready in {time.time() - t0:.1f}s ({n_lv} levels)")
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [ev() for _ in range(3)]
    marks[0].record()
    for ly in range(c.n_layers):
        c.build(ly)
    marks[1].record()
    for ly in range(c.n_layers):
        c.prefill(ly)
    marks[2].record()
    steps = [(ev(), ev()) for _ in range(c.steps)]
    for s_, (a, b) in enumerate(steps):
        a.record()
        c.decode(s_)
        b.record()
    torch.cuda.synchronize()
    for ly in range(c.n_layers):
        if torch.count_nonzero(R.decode_error_words(c.ws_dec, c.layers[ly]["tree"], wl.Hq)).item():
            raise RuntimeError("config 5: a decode step reported a timed-out wait")
    build_ms = marks[0].elapsed_time(marks[1])
    pre_ms = marks[1].elapsed_time(marks[2])
    dec_us = [a.elapsed_time(b) * 1e3 for a, b in steps]
    bb = build_bytes(c.L, Hkv, n_lv) * B * c.n_layers
    db = np.mean([decode_rows(c.t_dec + s_, 16, wl.k, n_lv)["rows"] for s_ in range(c.steps)]) \
        * ROW_BYTES * Hkv * B * c.n_layers
    med_us = sorted(dec_us)[len(dec_us) // 2]
    out = {
        "workload": f"{c.n_layers} layers, each 8 KV heads, 32 query heads, d=128, bf16, "
                    f"L={c.L}, C=16, k={wl.k}, own K/V/pooler: full build of every layer, a "
                    f"{T}-query causal chunk per layer, then {c.steps} decode steps (one new "
                    f"token per layer, fresh q/k/v, from t={c.t_dec})",
        "build_all_layers_ms": round(build_ms, 2),
        "build_GBs": round(bb / (build_ms * 1e-3) / 1e9, 1),
        "build_hbm_frac": round(bb / (build_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "prefill_all_layers_ms": round(pre_ms, 2),
        "prefill_tok_s": round(B * T / (pre_ms * 1e-3), 1),
        "decode_us_per_step_median": round(med_us, 2),
        "decode_us_per_step_mean": round(float(np.mean(dec_us)), 2),
        "decode_algorithmic_MB_per_step": round(db / 1e6, 1),
        "decode_hbm_frac": round(db / (med_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_steps": c.steps,
    }
    log("config 5: " + json.dumps(out))
    del c
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def measured_peaks():
    """This device's achievable rates, measured here: a 4 GiB device-to-device
    copy (bytes read + written per second) and an 8192^3 bf16 matrix product
    through torch (the vendor GEMM library), each the best of 10 timed
    runs."""
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)
    src = torch.empty(1 << 30, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    best_copy = 1e9
    for _ in range(10):
        a, b = ev(), ev()
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best_copy = min(best_copy, a.elapsed_time(b) * 1e-3)
    del src, dst
    n = 8192
    x = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    y = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    best_mm = 1e9
    for _ in range(10):
        a, b = ev(), ev()
        a.record()
        torch.matmul(x, y)
        b.record()
        torch.cuda.synchronize()
        best_mm = min(best_mm, a.elapsed_time(b) * 1e-3)
    del x, y
    torch.cuda.empty_cache()
    return {"copy_GBs": round(2 * (4 << 30) / best_copy / 1e9, 1),
            "bf16_gemm_TFLOPs": round(2 * n ** 3 / best_mm / 1e12, 1),
            "how": "best of 10: 4 GiB device copy (read + write); 8192^3 bf16 torch.matmul"}


def needle_recall_in_level0(w):
    """Fraction of the planted needles (decode slot 0's query) that the
    decode's selection reaches at level 0: needle tau is in A^(0) when its
    level-1 parent tau >> 4 is in S^(1).  A diagnostic of the random pooler,
    which is not trained to route."""
    import numpy as np
    tree = w.tree
    if tree.n_levels < 2 or w.needles.numel() == 0:
        return None
    sel = w.sel_dec.cpu().numpy().reshape(w.wl.B, tree.Hkv, tree.n_sel, tree.k)
    cnt = w.cnt_dec.cpu().numpy().reshape(w.wl.B, tree.Hkv, tree.n_sel)
    hit = tot = 0
    for b in range(w.wl.B):
        for j in range(tree.Hkv):
            s1 = set(sel[b, j, 0, : cnt[b, j, 0]].tolist())
            for tau in w.needles[b, j].tolist():
                hit += int((tau >> 4) in s1)
                tot += 1
    return round(hit / tot, 4)


SCRUB_BYTES = 512 << 20


COPY_BYTES = 512 << 20
# sources of the fused decode kernel: a counter summary counts only while
# their hash matches the one recorded with it
FUSED_SOURCES = ("long_context_kv_amd/csrc/decode_fused.hip", "long_context_kv_amd/csrc/recsa_common.hpp",
                 "long_context_kv_amd/csrc/recsa_device.hpp", "long_context_kv_amd/csrc/recsa_mfma.hpp",
                 "long_context_kv_amd/csrc/recsa_pool.hpp", "long_context_kv_amd/csrc/recsa_kernels.hpp",
                 "long_context_kv_amd/csrc/recsa_fused_ctl.hpp", "long_context_kv_amd/csrc/recsa_hw.hpp",
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


# CPU-baseline worker state, set in the parent before the pool forks (the
# workers read it copy-on-write; nothing of it is sent through pipes)
_CPU = {}


def _cpu_head_unit(j):
    """One KV head of the oracle baseline: tree build over the decode
    token's prefix, the decode walk + softmax (timed), then the exact-mode
    walk (not timed) for the agreement figure."""
    from threadpoolctl import threadpool_limits

    from oracle import recsa_oracle as O
    c = _CPU
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        Kt, Vt = O.build_tree(c["K0"][j], c["V0"][j], 16, c["n_levels"], c["P"], c["dtype"])
        t1 = time.perf_counter()
        qG = c["qd"][j * c["G"]:(j + 1) * c["G"]]
        _, tr = O.decode_reference(qG, c["t_dec"], Kt, Vt, 16, c["k"], c["cos"], c["sin"],
                                   c["dtype"])
        t2 = time.perf_counter()
        tr_x = O.walk(qG, c["t_dec"], Kt, 16, c["k"], exact=True, theta=c["theta"])
    sel = {l: lt.S for l, lt in tr.levels.items()}
    sel_x = {l: lt.S for l, lt in tr_x.levels.items()}
    upper = (Kt[1:], Vt[1:]) if j == 0 else None
    return j, t1 - t0, t2 - t1, sel, sel_x, upper


def _cpu_prefill_unit(i):
    """One prefill query of the chunk on KV head 0 (walk + softmax)."""
    from threadpoolctl import threadpool_limits

    from oracle import recsa_oracle as O
    c = _CPU
    t = c["L"] + int(i)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        Kt = [c["K0"][0][: t + 1]] + [x[: (t + 1) >> (4 * (l + 1))] for l, x in enumerate(c["Ku"])]
        Vt = [c["V0"][0][: t + 1]] + [x[: (t + 1) >> (4 * (l + 1))] for l, x in enumerate(c["Vu"])]
        O.decode_reference(c["qp"][i], t, Kt, Vt, 16, c["k"], c["cos"], c["sin"], c["dtype"])
        return time.perf_counter() - t0


def cpu_workers():
    """Worker processes for the CPU baseline: every core this process may run
    on, at most 16 (a one-GPU machine's CPU share)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def cpu_baseline(wl, tree, pdict, q_dec, q_pre, t_dec, L, T, sel_gpu):
    """The CPU oracle (NumPy float64, one BLAS thread per worker) on the
    host's cores, in processes over independent units, on a bounded sample of
    the same workload: every KV head's tree build over t_dec + 1 tokens and
    its decode walk + softmax at t_dec (one unit per head), then 256 evenly
    spaced queries of the prefill chunk on KV head 0, scaled to the chunk and
    to every head.  Also reported: the single-worker time per unit, and the
    agreement of the kernel's decode selection with the exact-arithmetic
    walk (no operand rounding, float64 RoPE) on the oracle's tree."""
    import multiprocessing as mp

    import numpy as np

    from oracle import recsa_oracle as O
    from tests import parity as PY

    heads = wl.Hkv * wl.B
    G = wl.Hq // wl.Hkv
    workers = cpu_workers()
    cos, sin = O.rope_table(wl.d, 16 * wl.k, wl.theta)
    _CPU.clear()
    _CPU.update(dict(
        K0=[PY.to64(tree.K[0][0, j, :t_dec + 1]) for j in range(wl.Hkv)],
        V0=[PY.to64(tree.V[0][0, j, :t_dec + 1]) for j in range(wl.Hkv)],
        P=PY.oracle_pooler(pdict), n_levels=tree.n_levels, dtype=wl.dtype, k=wl.k, G=G,
        t_dec=t_dec, qd=PY.to64(q_dec[0, 0]), cos=cos, sin=sin, theta=wl.theta, L=L))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(min(workers, wl.Hkv)) as pool:
        res = pool.map(_cpu_head_unit, range(wl.Hkv))
    t_heads = time.perf_counter() - t0
    res.sort(key=lambda r: r[0])
    build_1 = float(np.mean([r[1] for r in res]))
    dec_1 = float(np.mean([r[2] for r in res]))
    # exact-mode agreement of the kernel's selection (slot 0 decode query)
    same = tot = 0
    overlap = []
    for j, _, _, sel, sel_x, _ in res:
        for l, S in sel_x.items():
            g = np.sort(sel_gpu[0, j, l - 1][: len(sel[l])].cpu().numpy().astype(np.int64))
            tot += 1
            same += int(np.array_equal(g, S))
            overlap.append(len(set(g.tolist()) & set(S.tolist())) / max(len(S), 1))
    split_same = sum(int(np.array_equal(np.sort(sel_gpu[0, j, l - 1][: len(S)].cpu().numpy()), S))
                     for j, _, _, sel, _, _ in res for l, S in sel.items())
    # prefill sample on head 0
    Ku, Vu = res[0][5]
    _CPU.update(dict(Ku=Ku, Vu=Vu, qp=PY.to64(q_pre[0, :, :G])))
    idx = np.linspace(0, T - 1, 256).astype(int)
    t1 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        per_q = pool.map(_cpu_prefill_unit, idx.tolist())
    t_pre = time.perf_counter() - t1
    _CPU.clear()
    pre_1 = float(np.mean(per_q))
    # wall-clock rates on `workers` cores, scaled to the whole workload
    dec_wall = t_heads * dec_1 / (build_1 + dec_1)           # the decode share of the head units
    build_wall = t_heads - dec_wall
    pre_wall_chunk = t_pre * (T / len(idx)) * heads
    total = t_heads + t_pre
    log(f"cpu baseline ({total:.1f}s on {workers} workers): build/head {build_1:.2f}s, "
        f"decode/head {dec_1:.3f}s, prefill query/head {pre_1:.4f}s")
    return {
        "value": round(dec_wall * 1e6 * heads / wl.Hkv, 1), "unit": "us/token", "cores": workers,
        "kind": "oracle",
        "sample": (f"{wl.Hkv} KV head units on {min(workers, wl.Hkv)} worker processes "
                   f"(tree build over {t_dec + 1} tokens + decode walk/softmax at t={t_dec} "
                   f"each; value = the decode share of that wall time), then 256 evenly "
                   f"spaced queries of the {T}-query chunk on KV head 0 over {workers} workers, "
                   f"scaled x{T // 256} x{heads} heads; one BLAS thread per worker; "
                   f"{total:.1f}s of wall time"),
        "prefill_tok_s": round(B_T(wl, T) / pre_wall_chunk, 3),
        "build_full_ms": round(build_wall * 1e3, 1),
        "single_worker_s": {"build_per_head": round(build_1, 3), "decode_per_head": round(dec_1, 4),
                            "prefill_query_per_head": round(pre_1, 4)},
        "exact_mode_agreement": {
            "levels_identical": f"{same}/{tot}",
            "mean_overlap": round(float(np.mean(overlap)), 5) if overlap else None,
            "split_form_levels_identical": f"{split_same}/{tot}",
            "what": "decode query (slot 0), every KV head and scored level: the kernel's S^(l) "
                    "vs the walk in exact arithmetic (float64 RoPE at candidate-local "
                    "positions, no operand rounding) on the oracle's tree"},
    }


def B_T(wl, T):
    return wl.B * T


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
