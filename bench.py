#!/usr/bin/env python3
"""Benchmark of one block-sparse attention call on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
                    [--workload NAME] [--refresh-every R]

A step is one full call of the hot path on the workload's synthetic inputs
(already resident in HBM): block selection (pooling, scores, keep lists) and
block-sparse attention with compensation when the workload uses it, over
blocks of raster tokens or of the Hilbert order (read through the token
order inside the kernels: no separate reordering pass of Q, V or O).  The default
workload is the 1.3B-sized video layer (B=1, H=12, N=32760 tokens of a
21x30x52 latent grid, d=128, 128-token blocks, cumulative-mass 0.9 rule).

Printed: one JSON line.  ``value`` is the effective attention throughput in
TFLOP/s over the kept blocks (4*d*sum over kept block pairs of n_i*n_j)
divided by the whole step time; ``ms_per_step`` is that step time.
``roofline`` reports the attention kernel alone against the bf16 matrix-core
peak, timed with HIP events on the stream it is launched on.
``cpu_baseline`` times the CPU oracle on the same workload (whole, within a
time budget), with the tiny workload's oracle on one thread beside it.
Besides the headline workload the line carries (unless ``--no-extra``):
``cold_cache`` (the same call with a 512 MB device write before each call, so
the last-level cache holds none of the inputs), ``bandwidth`` (GB/s of the
pooling and Hilbert-permutation kernels, HIP events) and ``per_config`` (GPU
timings of every workload of the table: ms per call, selection and attention,
kept TFLOP and the attention kernel's fraction of the bf16 peak).
With ``--refresh-every R`` (mask reuse across calls) only every R-th call
selects; the others keep its mask and recompute only the compensation
centroids; the default R = 1 selects on every call.

Workloads with data-dependent blocks (``--workload wan13b_cocluster`` or
``wan13b_kmeans_comp``) time the clustered call instead: clustering of Q and
K, gathering Q, K, V into the padded clustered layout and the selection over
clusters (reported as ``ms_select``), the attention on that layout with token
counts per block, and the scatter of O back to token order.  Their kept work
counts true tokens only (padding excluded).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 matrix-core peak (256 CU x 2.4 GHz x 4096)
PEAK_HBM_GBS = 8000.0
ATTN_KERNEL = "k_bsattn_fwd"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_bsattn_fwd_wan13b_traffic.md")
ATTN_SOURCE = os.path.join(ROOT, "block_sparse_attention_hilbert_amd", "csrc", "k_attn.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(ATTN_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing, for another workload or for older kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = dict(re.findall(r"^- (\w+): (\S+)", text, flags=re.M))
    if fields.get("workload") != workload or fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, Q, K, V, budget_s: float = 40.0, tiny: bool = True):
    """The oracle (as it stands) on the workload: heads 0, 1, ... in turn,
    each one's full selection and float64 attention of all its query blocks,
    until done or the time budget is spent (the head in progress when it runs
    out is finished block by block up to the budget; the 1.3B-sized layer
    finishes whole in about 20 s on 16 cores).  Reported as kept-block TFLOP/s
    and wall time; with it, the tiny workload's oracle on one thread."""
    import oracle
    import workloads as W
    from threadpoolctl import threadpool_info

    t0 = time.perf_counter()
    perm = oracle.hilbert_perm(wl.T, wl.Hg, wl.W)[0] if wl.hilbert else None
    off = W.anchor_offset(wl.seed, 0, wl.nb)
    n = np.diff(oracle.block_bounds(wl.N, wl.block)).astype(np.float64)
    flops = 0.0
    heads = blocks = 0
    for h in range(wl.H):
        keep, _ = oracle.select_workload(wl, Q[:, h:h + 1], K[:, h:h + 1], heads=[h],
                                         anchor_offset=off, perm=perm,
                                         V=V[:, h:h + 1] if wl.rule == "err" else None)
        q, k, v = (oracle.bf16_to_f64(x[0, h]) for x in (Q, K, V))
        if perm is not None:
            q, k, v = (oracle.permute_tokens(x, perm) for x in (q, k, v))
        for i in range(wl.nb):
            oracle.attention_head(q, k, v, keep[0, 0], wl.block, wl.scale, comp=wl.comp,
                                  q_blocks=[i])
            flops += 4.0 * wl.d * n[i] * float((keep[0, 0, i] * n).sum())
            blocks += 1
            if time.perf_counter() - t0 > budget_s:
                break
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    whole = heads == wl.H and blocks == wl.H * wl.nb
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
           "kind": "oracle", "wall_s": round(dt, 2), "whole_workload": whole,
           "sample": (f"the whole workload: {wl.H} heads, selection + float64 attention of "
                      f"{blocks} query blocks ({dt:.1f} s wall)" if whole else
                      f"{heads} of {wl.H} heads of batch 0: selection + float64 attention of "
                      f"{blocks} query blocks ({dt:.1f} s wall)")}
    if tiny:
        out["tiny_one_thread"] = cpu_tiny_one_thread()
    return out


def cpu_tiny_one_thread():
    """The oracle on the tiny workload (selection + attention of every head)
    on one thread: wall time."""
    import oracle
    import workloads as W
    from threadpoolctl import threadpool_limits

    wl = W.WORKLOADS[1]
    Q, K, V = W.make_qkv(wl)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        keep, _ = oracle.select_workload(wl, Q, K)
        for h in range(wl.H):
            oracle.attention_head(oracle.bf16_to_f64(Q[0, h]), oracle.bf16_to_f64(K[0, h]),
                                  oracle.bf16_to_f64(V[0, h]), keep[0, h], wl.block, wl.scale)
        dt = time.perf_counter() - t0
    return {"workload": wl.name, "ms": round(dt * 1e3, 2), "cores": 1}


def cpu_baseline_clusters(wl, Q, K, V, budget_s: float = 15.0):
    """The clustered path's oracle on a bounded sample: heads in turn, each one's
    clustering and selection, then float64 attention of its query clusters one
    by one until the budget is spent.  Kept-token TFLOP/s of the sample."""
    import oracle
    from oracle import clusters as OC
    from oracle import tiles as OT
    from threadpoolctl import threadpool_info

    t0 = time.perf_counter()
    flops = 0.0
    heads = done = 0
    for h in range(wl.H):
        q, k, v = (oracle.bf16_to_f64(x[0, h]) for x in (Q, K, V))
        if wl.cluster == "tiles":
            ref = OT.tiles_workload_head(wl, q, k)
        else:
            ref = OC.cluster_workload_head(wl, q, k)
        kept_tok = ref["keepC"].astype(np.float64) @ ref["nk"].astype(np.float64)
        for a in range(wl.n_clusters):
            if ref["nq"][a] == 0:
                continue
            OC.cluster_attention_head(q, k, v, ref["aq"], ref["ak"], ref["keepC"], wl.scale,
                                      comp=wl.comp, q_clusters=[a])
            flops += 4.0 * wl.d * float(ref["nq"][a]) * float(kept_tok[a])
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads} of {wl.H} heads of batch 0: block formation + selection + float64 "
                      f"attention of {done} query clusters ({dt:.1f} s wall)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="workload number 1..5")
    ap.add_argument("--workload", default=None,
                    help="workload by name (overrides --config), e.g. wan13b_err")
    ap.add_argument("--refresh-every", type=int, default=1,
                    help="mask reuse: select on every r-th call only, the calls in between "
                         "keep the mask (compensation centroids still from their own K, V)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-per-workload", type=float, default=5.0,
                    help="seconds of oracle work per non-headline workload record")
    ap.add_argument("--cpu-budget", type=float, default=40.0,
                    help="seconds the CPU oracle baseline may take")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the headline workload: no cold-cache run, bandwidth legs or "
                         "per-workload records")
    ap.add_argument("--graph", action="store_true",
                    help="data-dependent blocks: time the calls as HIP graph replays "
                         "(stage times still come from eager calls)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path is data-parallel per head and query block; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W

    if args.calib_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 5}))
        return

    wl = W.by_name(args.workload) if args.workload else W.WORKLOADS[args.config]
    log(f"[bench] workload {wl.name}: generating inputs")
    Q, K, V = W.make_qkv(wl)

    def dev(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()

    Qd, Kd, Vd = dev(Q), dev(K), dev(V)
    if wl.cluster:
        return bench_clusters(args, wl, Q, K, V, Qd, Kd, Vd)
    res = time_calls(wl, Qd, Kd, Vd, args.steps, args.warmup, args.refresh_every)
    step_s, F_kept, keep = res["step_s"], res["F_kept"], res["keep"]
    fwd_s, sel_s = res["fwd_ms"] / 1e3, res["sel_ms"] / 1e3
    achieved = F_kept / fwd_s / 1e12
    traffic = read_traffic(wl.name)
    out = {
        "metric": "ms/attn call + effective TFLOP/s (kept blocks) at N=32760, H=12, d=128, 1 GPU",
        "value": round(F_kept / step_s / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded smooth-field video-latent Q/K, N(0,1) V)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d,
                   "latent_grid": [wl.T, wl.Hg, wl.W], "block": wl.block, "rule": wl.rule,
                   "mass": wl.mass if wl.rule == "mass" else None,
                   "density_kept": round(float(keep.mean()), 4),
                   "hilbert": wl.hilbert, "compensation": wl.comp,
                   "mask_refresh_every": args.refresh_every,
                   "parallelism": "single GPU"},
        "ms_select": round(sel_s * 1e3, 4),
        "selections_timed": res["selections"],
        "ms_attention": round(fwd_s * 1e3, 4),
        "ms_attention_prepare": round(res["prep_ms"], 4),
        "select_over_attention": round(sel_s / fwd_s, 4),
        "kept_tflop_per_call": round(F_kept / 1e12, 4),
        "roofline": {"bound": "mfma", "kernel": ATTN_KERNEL, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    if not args.no_extra:
        log("[bench] cold calls (a 512 MB write between calls flushes the last-level cache)")
        cold = time_calls(wl, Qd, Kd, Vd, 10, 2, args.refresh_every, flush_bytes=512 << 20)
        out["cold_cache"] = {"ms_per_call": round(cold["call_ms"], 4),
                             "ms_attention": round(cold["fwd_ms"], 4),
                             "ms_select": round(cold["sel_ms"], 4),
                             "flush": "512 MB device write before each call, outside the timing"}
        out["bandwidth"] = bandwidth_legs()
        out["per_config"] = per_config_records(args, wl, res)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle as it stands, the whole workload)")
        out["cpu_baseline"] = cpu_baseline(wl, Q, K, V, budget_s=args.cpu_budget)
    print(json.dumps(out), flush=True)


def time_calls(wl, Qd, Kd, Vd, steps, warmup, refresh_every=1, flush_bytes=0):
    """Times `steps` calls of the path on resident inputs after `warmup`
    untimed ones: the wall time of the back-to-back calls, synchronised on both
    sides, and HIP events on the launch stream around selection, preparation,
    attention and the whole call (means).  With ``flush_bytes`` a device
    buffer of that size is written before every call (outside the events) to
    flush the last-level cache; the wall time then includes the flushes."""
    import torch
    import block_sparse_attention_hilbert_amd as sa
    from block_sparse_attention_hilbert_amd.pipeline import BlockSparseAttention
    import workloads as W

    pipe = BlockSparseAttention(sa.problem_for(wl), sa.spec_for(wl), hilbert=wl.hilbert,
                                refresh_every=refresh_every)
    stream = torch.cuda.current_stream()
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda") if flush_bytes else None
    selected = []

    def step(call_idx, ev):
        if flush is not None:
            flush.fill_(call_idx & 255)
        off = W.anchor_offset(wl.seed, call_idx, wl.nb) if wl.n_anchors else None
        reuse = pipe.reuses_next()
        selected.append(not reuse)
        ev[0].record(stream)
        ev[1].record(stream)
        if reuse:
            pipe.run_centroids(Kd, Vd)
        else:
            pipe.run_select(Qd, Kd, Vd, off)
        ev[2].record(stream)
        pipe.run_fwd_prepare(Vd)
        ev[3].record(stream)
        pipe.run_fwd_attention(Qd, Kd)
        ev[4].record(stream)
        ev[5].record(stream)
        pipe.calls += 1

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(max(steps, 1))]
    log(f"[bench] {wl.name}: warmup {warmup}")
    for i in range(warmup):
        step(i, events[0])
    torch.cuda.synchronize()
    # timed region: exactly `steps` back-to-back calls, synchronised on both sides
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, events[i])
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    ev = events[:steps]
    mean = lambda a, b: float(np.mean([e[a].elapsed_time(e[b]) for e in ev]))
    log(f"[bench] {wl.name}: {steps} steps: {step_s * 1e3:.3f} ms/step")
    # kept work of the last call's mask (only the rotating anchors change it
    # from call to call)
    keep = pipe.keep_mask()
    n = np.diff(np.append(np.arange(wl.nb) * wl.block, wl.N)).astype(np.float64)
    F_kept = 4.0 * wl.d * float((keep * np.outer(n, n)).sum())
    res = {"step_s": step_s, "F_kept": F_kept, "keep": keep,
           "sel_ms": mean(1, 2), "prep_ms": mean(2, 3), "fwd_ms": mean(3, 4),
           "call_ms": mean(0, 5), "selections": int(sum(selected[warmup:]))}
    del pipe, flush
    torch.cuda.empty_cache()
    return res


def per_config_records(args, main_wl, main_res):
    """One record per workload of the table, plus the reported-only LVSA point
    at a ±4-frame window (the structure closest to the page's ~8 % density):
    GPU timings and, unless the CPU baseline is off, the oracle's rate on a
    bounded sample of the same workload (inputs made and freed one workload at
    a time)."""
    import torch
    import workloads as W

    recs = []
    table = [(c, W.WORKLOADS[c]) for c in sorted(W.WORKLOADS)] + [(None, W.by_name("lvsa_6x_r4"))]
    for c, wl in table:
        Q, K, V = W.make_qkv(wl)
        if wl.name == main_wl.name:
            r = main_res
        else:
            dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
            Qd, Kd, Vd = dev(Q), dev(K), dev(V)
            r = time_calls(wl, Qd, Kd, Vd, 10, 2)
            del Qd, Kd, Vd
            torch.cuda.empty_cache()
        cpu = None
        if not args.no_cpu_baseline and wl.name != main_wl.name:
            # the headline workload's oracle runs whole in cpu_baseline
            log(f"[bench] oracle sample: {wl.name}")
            b = cpu_baseline(wl, Q, K, V, budget_s=args.cpu_budget_per_workload, tiny=False)
            cpu = {k: b[k] for k in ("value", "unit", "cores", "wall_s", "whole_workload", "sample")}
        del Q, K, V
        att = r["F_kept"] / (r["fwd_ms"] / 1e3) / 1e12
        rec = {"config": c, "workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N,
                     "block": wl.block, "rule": wl.rule,
                     "density_kept": round(float(r["keep"].mean()), 4),
                     "ms_per_call": round(r["step_s"] * 1e3, 4),
                     "ms_select": round(r["sel_ms"], 4),
                     "ms_attention": round(r["fwd_ms"], 4),
                     "select_over_attention": round(r["sel_ms"] / r["fwd_ms"], 4),
                     "kept_tflop_per_call": round(r["F_kept"] / 1e12, 4),
                     "tflops_call": round(r["F_kept"] / r["step_s"] / 1e12, 2),
                     "tflops_attention": round(att, 2),
                     "frac": round(att / PEAK_BF16_TFLOPS, 4)}
        if c is None:
            rec["reported_only"] = "window ±4 latent frames + 4 anchors (the ±1-frame table entry keeps 2.7 %)"
        if cpu is not None:
            rec["cpu_oracle"] = cpu
        recs.append(rec)
    return recs


def bandwidth_legs():
    """Achieved bandwidth of the pooling and reordering kernels on the
    1.3B-sized layer's shape (one call each, HIP events, mean of 20):
    pooling = the block means of K and block sums of V (sparse_attn_centroids,
    the same kernel the selection runs on Q and K: reads two [1,12,32760,128]
    bf16 tensors, writes fp32 block statistics); reordering = one Hilbert
    permutation of one tensor (read + write)."""
    import torch
    import block_sparse_attention_hilbert_amd as sa
    import workloads as W

    wl = W.WORKLOADS[2]
    prob = sa.problem_for(wl)
    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    Q, K, V = W.make_qkv(wl)
    Kd, Vd = dev(K), dev(V)
    km = torch.empty(wl.B, wl.H, wl.nb, wl.d, dtype=torch.float32, device="cuda")
    vs = torch.empty_like(km)
    perm = torch.from_numpy(sa.hilbert_perm_build(wl.T, wl.Hg, wl.W)[0]).cuda()
    dst = torch.empty_like(Kd)

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    tensor_bytes = wl.B * wl.H * wl.N * wl.d * 2
    stats_bytes = 2 * wl.B * wl.H * wl.nb * wl.d * 4
    pool_ms = timed(lambda: sa.centroids(prob, Kd, Vd, km, vs))
    perm_ms = timed(lambda: sa.hilbert_permute(prob, Kd, perm, dst))
    pool_b, perm_b = 2 * tensor_bytes + stats_bytes, 2 * tensor_bytes
    return {"pooling": {"kernel": "k_pool", "ms": round(pool_ms, 4), "bytes": pool_b,
                        "gbs": round(pool_b / pool_ms / 1e6, 1),
                        "frac": round(pool_b / pool_ms / 1e6 / PEAK_HBM_GBS, 4)},
            "permute": {"kernel": "k_permute", "ms": round(perm_ms, 4), "bytes": perm_b,
                        "gbs": round(perm_b / perm_ms / 1e6, 1),
                        "frac": round(perm_b / perm_ms / 1e6 / PEAK_HBM_GBS, 4)},
            "workload": wl.name, "peak_gbs": PEAK_HBM_GBS}


def bench_clusters(args, wl, Q, K, V, Qd, Kd, Vd):
    import torch
    import block_sparse_attention_hilbert_amd as sa
    from block_sparse_attention_hilbert_amd.pipeline import ClusteredAttention

    pipe = ClusteredAttention(sa.problem_for(wl), sa.cluster_spec_for(wl), sa.spec_for(wl),
                              refresh_every=args.refresh_every)
    stream = torch.cuda.current_stream()
    selected = []

    def step(ev):
        reuse = pipe.reuses_next()
        selected.append(not reuse)
        ev[0].record(stream)
        if not reuse:
            pipe.run_cluster(Qd, Kd, Vd)
        ev[1].record(stream)
        pipe.run_gather(Qd, Kd, Vd)
        if reuse:
            pipe.run_centroids()
        else:
            pipe.run_select()
        ev[2].record(stream)
        pipe.run_fwd_prepare()
        ev[3].record(stream)
        pipe.run_fwd_attention()
        ev[4].record(stream)
        pipe.run_scatter()
        pipe.calls += 1

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
              for _ in range(max(args.steps, 1))]
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step(events[0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    ev = events[: args.steps]
    cl_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    gs_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    prep_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    fwd_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in ev]))
    log(f"[bench] {args.steps} steps: {step_s * 1e3:.3f} ms/step")
    eager_s = step_s
    if args.graph:
        from block_sparse_attention_hilbert_amd.pipeline import GraphedCall
        graphed = GraphedCall(pipe, Qd, Kd, Vd)
        for _ in range(args.warmup):
            graphed()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graphed()
        torch.cuda.synchronize()
        step_s = (time.perf_counter() - t0) / args.steps
        log(f"[bench] {args.steps} graph replays: {step_s * 1e3:.3f} ms/step")
    # kept work in true tokens: q tokens of each padded query block times the
    # key tokens of the blocks it keeps
    kept = pipe.kept_tokens().cpu().numpy().astype(np.float64)
    qcnt = pipe.cl.q_cnt.reshape(-1).cpu().numpy().astype(np.float64)
    F_kept = 4.0 * wl.d * float((qcnt * kept).sum())
    slots = float(pipe.pprob.N) * wl.B * wl.H
    fwd_s = fwd_ms / 1e3
    achieved = F_kept / fwd_s / 1e12
    sel_s = (cl_ms + gs_ms) / 1e3
    out = {
        "metric": "ms/attn call + effective TFLOP/s (kept blocks) at N=32760, H=12, d=128, 1 GPU",
        "value": round(F_kept / step_s / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded smooth-field video-latent Q/K, N(0,1) V)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d,
                   "latent_grid": [wl.T, wl.Hg, wl.W], "block": wl.block, "rule": wl.rule,
                   "mass": wl.mass if wl.rule == "mass" else None,
                   "cluster": wl.cluster, "n_clusters": wl.n_clusters,
                   "cluster_iters": wl.cluster_iters, "padded_blocks": pipe.nbp,
                   "token_density_kept": round(float((qcnt * kept).sum()) /
                                               (wl.B * wl.H * float(wl.N) ** 2), 4),
                   "padding_fraction": round(1.0 - wl.B * wl.H * wl.N / slots, 4),
                   "compensation": wl.comp, "partition_refresh_every": args.refresh_every,
                   "launch": "hip graph replay" if args.graph else "eager",
                   "parallelism": "single GPU"},
        "tile_shape_per_head": (None if pipe.shape_idx is None else
                                [list(wl.tile_shapes[i]) for i in pipe.shape_idx.cpu().tolist()]),
        "clusterings_timed": int(sum(selected[args.warmup:])),
        "ms_per_step_eager": round(eager_s * 1e3, 4),
        "ms_cluster": round(cl_ms, 4),
        "ms_gather_select": round(gs_ms, 4),
        "ms_select": round(sel_s * 1e3, 4),
        "ms_attention": round(fwd_ms, 4),
        "ms_attention_prepare": round(prep_ms, 4),
        "select_over_attention": round(sel_s / fwd_s, 4),
        "kept_tflop_per_call": round(F_kept / 1e12, 4),
        "roofline": {"bound": "mfma", "kernel": ATTN_KERNEL, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(wl.name)},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle, bounded sample)")
        out["cpu_baseline"] = cpu_baseline_clusters(wl, Q, K, V)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
