#!/usr/bin/env python3
"""Benchmark of the paged-KV decode hot path on one MI355X.

A step is one decode step of a Qwen3-4B-like model's attention over all 36
layers: ``pkv_plan`` walks the step's page table once, then for each layer
``pkv_run`` appends the batch's new K/V rows and decodes one query row per
entry (batch 64, 32 query / 8 KV heads, head_dim 128, page_size 16, lengths
log-uniform in [64, 4096]).  Inputs are seeded synthetic data resident in HBM
before timing starts.  The step is captured once as a HIP graph and replayed.

Printed: ONE JSON line with the whole-step throughput (algorithmic bytes per
second), the decode kernel's roofline figures measured live with HIP events on
its own stream, and the fp64 oracle timed on the host cores on a bounded
sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--config C] [--batch B]
                  [--chunk-pages P] [--no-cpu-baseline] [--no-check] [--probe-copy]

The other workloads (--config 1, 2, 4, 5; --batch for the batch sweep of the
Qwen3-0.6B-like one) print the same line for that workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores, published
METRIC = "paged decode attention: achieved HBM GB/s (% of peak) + decode rows/sec"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--batch", type=int, default=0,
                    help="batch size (with its padding share) instead of the workload's own")
    ap.add_argument("--chunk-pages", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="approximate CPU time (summed over threads) of the oracle sample")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--separate", action="store_true",
                    help="per layer pkv_append then a decode-only pkv_run")
    ap.add_argument("--plan-per-layer", action="store_true",
                    help="per layer pkv_append_decode (plans inside every call)")
    ap.add_argument("--qk-norm-rope", action="store_true",
                    help="per layer the fused q/k RMSNorm + rotary + KV write, then a "
                         "decode-only pkv_run on its q")
    ap.add_argument("--mrope", action="store_true",
                    help="with --qk-norm-rope or --fused-norm-rope: multimodal RoPE "
                         "(positions (L-1, (L-1)/2, "
                         "(L-1)/3), contiguous 24:20:20 bands of pairs)")
    ap.add_argument("--fused-norm-rope", action="store_true",
                    help="per layer one pkv_run_qk_norm_rope: the decode with the append "
                         "and the q/k RMSNorm + rotary folded in")
    ap.add_argument("--prefill", action="store_true",
                    help="a mixed step instead: decode rows plus whole new prompts, per "
                         "layer pkv_prefill (append + causal attention)")
    ap.add_argument("--prompt-rows", type=int, default=512,
                    help="rows of each new prompt in the mixed step")
    ap.add_argument("--decode-rows", type=int, default=60,
                    help="decode entries (one row each) in the mixed step")
    ap.add_argument("--one-call", action="store_true",
                    help="mixed step as one pkv_mixed_run per layer over all entries, on "
                         "one pkv_plan_mixed per step (default: the decode entries through "
                         "pkv_plan + pkv_run, the prompts through pkv_prefill, on two "
                         "tables)")
    ap.add_argument("--probe-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter scale)")
    return ap.parse_args()


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when the kernel source changed since they were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)
        with open(os.path.join(ROOT, rec["kernel_source"]), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    if not sha.startswith(rec["source_sha256_prefix"]):
        return None
    return rec["launch_read_bytes"] + rec["launch_write_bytes"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def probe_copy(torch, quiet=False):
    """Plain device-to-device copy of a known size: the counter calibration,
    and the copy rate the chip reaches (an informational ceiling)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 20
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    rec = {"probe": "copy", "bytes_read": n, "bytes_written": n, "ms": dt * 1e3,
           "GBs": 2 * n / dt / 1e9}
    del src, dst
    torch.cuda.empty_cache()
    if not quiet:
        print(json.dumps(rec), flush=True)
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.probe_copy:
        probe_copy(torch)
        return 0
    if args.prefill:
        return bench_prefill(args, torch)

    import paged_kv_decode_pkv_amd as pkv
    import workloads

    spec = workloads.CONFIGS[args.config]
    table = workloads.make_table(spec, args.batch or None)
    nl, b = spec.num_layers, table.batch
    hq, hkv, d, ps = spec.num_qo_heads, spec.num_kv_heads, spec.head_dim, spec.page_size
    dev = torch.device("cuda:0")
    log(f"workload {spec.name}: batch {b}, layers {nl}, pool {table.num_pages} pages, "
        f"max pages/entry {table.max_pages_per_req}")

    # ---- inputs, resident in HBM before timing
    cache = torch.zeros((nl, table.num_pages, 2, ps, hkv, d), dtype=torch.bfloat16,
                        device=dev)
    Q = torch.empty((nl, b, hq, d), dtype=torch.bfloat16, device=dev)
    KN = torch.empty((nl, b, hkv, d), dtype=torch.bfloat16, device=dev)
    VN = torch.empty_like(KN)
    offs = workloads.k_offsets(spec)
    for layer in range(nl):
        q, kn, vn = workloads.draw_layer_device(cache[layer], table,
                                                [1000 * spec.cfg + layer, b], hq,
                                                spec.sigma, offs,
                                                real_head_dim=spec.real_head_dim)
        Q[layer], KN[layer], VN[layer] = q, kn, vn
    tabs = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)
            for x in (table.indptr, table.indices, table.last_len)]
    out = torch.empty((nl, b, hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((nl, b, hq), dtype=torch.float32, device=dev)
    nr = None
    if args.qk_norm_rope or args.fused_norm_rope:
        # per-layer RMSNorm weights, the new tokens' positions, the rotated q
        gen = torch.Generator(device=dev).manual_seed(1000 * spec.cfg + 997)
        nr = {"qw": (torch.rand((nl, d), generator=gen, device=dev) + 0.5).to(torch.bfloat16),
              "kw": (torch.rand((nl, d), generator=gen, device=dev) + 0.5).to(torch.bfloat16),
              "pos": torch.from_numpy((table.lengths - 1).astype(np.int32)).to(dev),
              "qo": torch.empty_like(Q), "eps": 1e-6, "theta": 1e6}
        if args.mrope:
            if not (args.qk_norm_rope or args.fused_norm_rope):
                raise SystemExit("--mrope goes with --qk-norm-rope or --fused-norm-rope")
            last = (table.lengths - 1).astype(np.int32)
            nr["pos3"] = torch.from_numpy(
                np.stack([last, last // 2, last // 3], axis=1).astype(np.int32)).to(dev)
            h = d // 2
            t3, h3 = h * 24 // 64, h * 20 // 64
            nr["axis"] = np.array([0] * t3 + [1] * h3 + [2] * (h - t3 - h3), np.uint8)
    maxp = table.max_pages_per_req
    chunk = args.chunk_pages
    ws_bytes = pkv.workspace_size(pkv.cache_desc(cache), hq, b, maxp, chunk)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"inputs resident: cache {cache.numel() * 2 / 2**30:.1f} GiB, "
        f"chunk {chunk} pages, workspace {ws_bytes / 2**20:.1f} MiB")

    # ---- pre-marshalled C-ABI calls (the binding's arguments, built once)
    desc = pkv.cache_desc(cache)
    vp = ctypes.c_void_p
    tab_ptrs = [vp(t.data_ptr()) for t in tabs]
    null = vp(0)
    ws_args = (vp(ws.data_ptr()), ws.numel())

    def calls_for(stream_handle):
        """(plan call or None, per-layer [(fn, args, name), ...])"""
        s = vp(stream_handle)
        plan = None
        if not args.plan_per_layer:
            plan = (desc, hq, *tab_ptrs, b, maxp, chunk, *ws_args, s)
        layers = []
        for layer in range(nl):
            kn, vn = vp(KN[layer].data_ptr()), vp(VN[layer].data_ptr())
            qo = (vp(Q[layer].data_ptr()), hq)
            res = (ctypes.c_float(spec.sm_scale), vp(out[layer].data_ptr()),
                   vp(lse[layer].data_ptr()), maxp, chunk, *ws_args, s)
            cl = []
            if args.fused_norm_rope:
                head = (vp(cache.data_ptr()), desc, layer, kn, vn, *qo, b,
                        vp(nr["qw"][layer].data_ptr()), vp(nr["kw"][layer].data_ptr()),
                        ctypes.c_float(nr["eps"]), ctypes.c_float(nr["theta"]))
                if "axis" in nr:
                    cl.append((pkv.lib.pkv_run_qk_norm_mrope,
                               (*head, vp(nr["pos3"].data_ptr()),
                                nr["axis"].ctypes.data_as(vp), *res), "pkv_run_qk_norm_mrope"))
                else:
                    cl.append((pkv.lib.pkv_run_qk_norm_rope,
                               (*head, vp(nr["pos"].data_ptr()), *res),
                               "pkv_run_qk_norm_rope"))
            elif args.qk_norm_rope:
                qo = (vp(nr["qo"][layer].data_ptr()), hq)
                head = (vp(cache.data_ptr()), desc, layer, vp(Q[layer].data_ptr()), hq, kn,
                        vn, vp(nr["qw"][layer].data_ptr()), vp(nr["kw"][layer].data_ptr()),
                        ctypes.c_float(nr["eps"]), ctypes.c_float(nr["theta"]))
                tail = (*tab_ptrs, b, vp(nr["qo"][layer].data_ptr()), s)
                if "axis" in nr:
                    cl.append((pkv.lib.pkv_qk_norm_mrope_append,
                               (*head, vp(nr["pos3"].data_ptr()),
                                nr["axis"].ctypes.data_as(vp), *tail),
                               "pkv_qk_norm_rope_append"))
                else:
                    cl.append((pkv.lib.pkv_qk_norm_rope_append,
                               (*head, vp(nr["pos"].data_ptr()), *tail),
                               "pkv_qk_norm_rope_append"))
                cl.append((pkv.lib.pkv_run, (vp(cache.data_ptr()), desc, layer, null, null,
                                             *qo, b, *res), "pkv_run"))
            elif args.separate:
                cl.append((pkv.lib.pkv_append,
                           (vp(cache.data_ptr()), desc, layer, kn, vn, *tab_ptrs, b, s),
                           "pkv_append"))
                cl.append((pkv.lib.pkv_run, (vp(cache.data_ptr()), desc, layer, null, null,
                                             *qo, b, *res), "pkv_run"))
            elif args.plan_per_layer:
                cl.append((pkv.lib.pkv_append_decode,
                           (vp(cache.data_ptr()), desc, layer, kn, vn, *qo, *tab_ptrs, b,
                            *res), "pkv_append_decode"))
            else:
                cl.append((pkv.lib.pkv_run, (vp(cache.data_ptr()), desc, layer, kn, vn,
                                             *qo, b, *res), "pkv_run"))
            layers.append(cl)
        return plan, layers

    if args.fused_norm_rope and args.mrope:
        call_name = "pkv_run_qk_norm_mrope (norm + multimodal rotary + append + decode)"
    elif args.fused_norm_rope:
        call_name = "pkv_run_qk_norm_rope (norm + rotary + append + decode)"
    elif args.qk_norm_rope and args.mrope:
        call_name = "pkv_qk_norm_mrope_append + pkv_run"
    elif args.qk_norm_rope:
        call_name = "pkv_qk_norm_rope_append + pkv_run"
    elif args.separate:
        call_name = "pkv_append + pkv_run"
    elif args.plan_per_layer:
        call_name = "pkv_append_decode"
    else:
        call_name = "pkv_run (append + decode)"

    def run_step(plan, layers, events=None):
        if plan is not None:
            rc = pkv.lib.pkv_plan(*plan)
            if rc:
                raise pkv.PkvError(rc, "pkv_plan")
        for layer in range(nl):
            for i, (fn, a, name) in enumerate(layers[layer]):
                timed = events is not None and i == len(layers[layer]) - 1
                if timed:
                    events[layer][0].record()
                rc = fn(*a)
                if rc:
                    raise pkv.PkvError(rc, name)
                if timed:
                    events[layer][1].record()

    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        plan_call, layer_calls = calls_for(stream.cuda_stream)
        for _ in range(2):
            run_step(plan_call, layer_calls)
    torch.cuda.synchronize()

    # ---- the step as one HIP graph
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            cplan, clayers = calls_for(cap.cuda_stream)
            run_step(cplan, clayers)
        torch.cuda.synchronize()

    def replay():
        if graph is not None:
            graph.replay()
        else:
            run_step(plan_call, layer_calls)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            replay()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    with torch.cuda.stream(stream):
        # an event between consecutive steps: per-step durations as well
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(args.steps):
            replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_step_ev = ev[0].elapsed_time(ev[-1]) / args.steps
    step_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    p10, p50, p90 = (float(x) for x in np.percentile(step_ms, [10, 50, 90]))
    log(f"step: {ms_step:.4f} ms wall, {ms_step_ev:.4f} ms events "
        f"(p10 {p10:.4f}, median {p50:.4f}, p90 {p90:.4f})")

    # ---- live per-launch timing of the decode kernel: a HIP graph of the
    # step's per-layer launches alone (no plan), replayed between two events
    # recorded on the stream the kernels run on; a launch's duration is the
    # elapsed time over the launches, so it includes the dispatch gap to the
    # next launch (rocprofv3's kernel time leaves that gap out).  Workloads of
    # few layers repeat their layers in the graph (at least 32 launches), so
    # the host's graph submissions do not leave the GPU idle between them;
    # a repeated launch recomputes the same outputs.
    ksteps = max(1, min(args.steps, 20))
    reps = -(-32 // nl)
    run_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(run_graph):
        _, rlayers = calls_for(torch.cuda.current_stream().cuda_stream)
        # the decode launches only (with --separate, not the appends)
        rlayers = [[c for c in cl if c[2] not in ("pkv_append", "pkv_qk_norm_rope_append")]
                   for cl in rlayers]
        for _ in range(reps):
            run_step(None, rlayers)
    torch.cuda.synchronize()
    launches_per_step = reps * sum(len(c) for c in rlayers)
    with torch.cuda.stream(stream):
        for _ in range(2):
            run_graph.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(ksteps):
            run_graph.replay()
        g1.record()
    torch.cuda.synchronize()
    dec_us = g0.elapsed_time(g1) * 1e3 / (ksteps * launches_per_step)
    # the same launches issued one by one, an event pair around each (adds
    # the host launch path to every launch): reported alongside
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(nl)] for _ in range(ksteps)]
    with torch.cuda.stream(stream):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(20_000_000)   # let the host queue run ahead of the GPU
        for k in range(ksteps):
            run_step(plan_call, layer_calls, events=evs[k])
    torch.cuda.synchronize()
    durs = np.array([[a.elapsed_time(z) for a, z in row] for row in evs]) * 1e3   # us
    eager_us = float(durs.mean())

    copy = probe_copy(torch, quiet=True)
    log(f"plain 1 GiB device copy: {copy['GBs']:.0f} GB/s (read + write)")

    nr_us = None
    if args.qk_norm_rope:
        # the fused norm/rotary/KV-write launches alone, timed the same way
        nr_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(nr_graph):
            _, nlayers = calls_for(torch.cuda.current_stream().cuda_stream)
            nlayers = [[c for c in cl if c[2] == "pkv_qk_norm_rope_append"] for cl in nlayers]
            for _ in range(reps):
                run_step(None, nlayers)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(2):
                nr_graph.replay()
            n0, n1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n0.record()
            for _ in range(ksteps):
                nr_graph.replay()
            n1.record()
        torch.cuda.synchronize()
        nr_us = n0.elapsed_time(n1) * 1e3 / (ksteps * reps * nl)

    by = workloads.algorithmic_bytes(table, hq, hkv, d)
    if args.fused_norm_rope:
        step_bytes = nl * by["fused_norm_rope"]
    else:
        step_bytes = nl * (by["decode"] + by["norm_rope"] if args.qk_norm_rope else by["total"])
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    rows_per_s = int(table.active.sum()) / (ms_step * 1e-3)
    launch_bytes = by["decode"] if (args.separate or args.qk_norm_rope) else by["total"]
    if args.fused_norm_rope:
        launch_bytes = by["fused_norm_rope"]
    dec_gbs = launch_bytes / (dec_us * 1e-6) / 1e9
    log(f"decode launch avg {dec_us:.2f} us (graph; eager with events {eager_us:.2f} us) "
        f"-> {dec_gbs:.0f} GB/s algorithmic; step {gbs:.0f} GB/s")

    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec.name, "batch": b, "active": int(table.active.sum()),
                   "layers": nl, "num_qo_heads": hq, "num_kv_heads": hkv, "head_dim": d,
                   "page_size": ps,
                   "lengths": ("log-uniform" if spec.length_dist == "loguniform" else "uniform")
                   + f" [{spec.length_lo}, {spec.length_hi}]",
                   "head_dim_real": spec.real_head_dim or d,
                   "paired_streams": spec.paired,
                   "kv_chunk_pages": chunk, "hip_graph": graph is not None,
                   "call": call_name,
                   "step_bytes": step_bytes},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "decode_rows_per_s": round(rows_per_s, 1),
        "ms_per_step_events": round(ms_step_ev, 5),
        "ms_per_step_p10_median_p90": [round(p10, 5), round(p50, 5), round(p90, 5)],
        "gbs_at_median_step": round(step_bytes / (p50 * 1e-3) / 1e9, 1),
        "copy_probe_gbs": round(copy["GBs"], 1),
        "roofline": {"bound": "hbm", "kernel": f"{call_name}: run_kernel (decode + merge)",
                     "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if args.config == 3 and not args.separate
                     and not args.plan_per_layer and not args.qk_norm_rope
                     and not args.fused_norm_rope
                     and args.chunk_pages == 0 else None,
                     "bytes_per_launch": launch_bytes, "avg_launch_us": round(dec_us, 3),
                     "launches": int(ksteps * launches_per_step),
                     "timing": "HIP events around graph replays of the step's run launches, layers "
                               "repeated to at least 32 launches "
                               "(no plan); per launch = elapsed / launches",
                     "avg_launch_us_eager_events": round(eager_us, 3)},
    }

    if nr_us is not None:
        result["norm_rope"] = {
            "kernel": ("pkv_qk_norm_mrope_append: norm_rope_kernel<D, true>" if "axis" in nr
                       else "pkv_qk_norm_rope_append: norm_rope_kernel"),
            "avg_launch_us": round(nr_us, 3), "bytes_per_launch": by["norm_rope"],
            "achieved_gbs": round(by["norm_rope"] / (nr_us * 1e-6) / 1e9, 1),
            "bound": "latency",
            "note": "a few bytes per entry and head: the launch is bound by latency"}
        log(f"norm_rope launch avg {nr_us:.2f} us")
    if not args.no_check:
        result["parity"] = check_sample(spec, table, cache, Q, KN, VN, out, lse, torch, nr)
        log(f"parity on sampled rows: {result['parity']}")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, table, cache, Q, KN, VN, torch,
                                              args.cpu_seconds)
        if nr_us is not None:
            result["norm_rope"]["cpu_oracle"] = norm_rope_oracle_time(table, Q, KN, VN, nr,
                                                                      by["norm_rope"])
    print(json.dumps(result), flush=True)
    return 0


def bench_prefill(args, torch):
    """Mixed step on the Qwen3-4B-like shape: 60 decode rows (the first 60
    entries of the batch-64 workload, one row each) plus 4 new prompts of
    ``--prompt-rows`` rows that fill their entries; per layer one pkv_prefill
    (append of every new row, causal attention of every row), 36 layers,
    captured as one HIP graph."""
    import paged_kv_decode_pkv_amd as pkv
    import workloads
    spec = workloads.CONFIGS[3]
    base = workloads.make_table(spec)
    nd, npr, pr = int(args.decode_rows), 4, int(args.prompt_rows)
    lengths = np.concatenate([base.lengths[:nd], np.full(npr, pr)])
    nrows = np.concatenate([np.ones(nd, np.int64), np.full(npr, pr)])
    rng = np.random.default_rng([1000 * spec.cfg + 996, pr])
    table = workloads.table_from_lengths(lengths, np.ones(len(lengths), bool),
                                         spec.page_size, None, rng)
    nl, hq, hkv, d, ps = (spec.num_layers, spec.num_qo_heads, spec.num_kv_heads,
                          spec.head_dim, spec.page_size)
    b = table.batch
    qo_h = np.concatenate([[0], np.cumsum(nrows)]).astype(np.int32)
    rows = int(qo_h[-1])
    dev = torch.device("cuda:0")
    log(f"mixed step: {nd} decode rows + {npr} prompts of {pr} rows = {rows} rows, "
        f"{nl} layers, pool {table.num_pages} pages")
    cache = torch.zeros((nl, table.num_pages, 2, ps, hkv, d), dtype=torch.bfloat16,
                        device=dev)
    gen = torch.Generator(device=dev).manual_seed(1000 * spec.cfg + 995)
    Q = torch.randn((nl, rows, hq, d), generator=gen, device=dev).to(torch.bfloat16)
    KN = torch.randn((nl, rows, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    VN = torch.randn((nl, rows, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    for layer in range(nl):
        workloads.draw_layer_device(cache[layer], table, [1000 * spec.cfg + 900 + layer, b],
                                    hq, spec.sigma)
    tabs = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)
            for x in (table.indptr, table.indices, table.last_len)]
    qo = torch.from_numpy(qo_h).to(dev)
    out = torch.empty((nl, rows, hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((nl, rows, hq), dtype=torch.float32, device=dev)
    maxr = int(nrows.max())
    split = nd > 0 and not args.one_call
    mixed = nd > 0 and args.one_call
    dmaxp = int(max((table.indptr[e + 1] - table.indptr[e] for e in range(nd)), default=1))
    if mixed:
        # one table, one plan per step over the rows: decode rows on the
        # decode's schedule, prompts through the prefill, per layer one call
        mws = torch.empty(max(pkv.workspace_size(pkv.cache_desc(cache), hq, rows, dmaxp, 0),
                              256), dtype=torch.uint8, device=dev)
    if split:
        # the decode entries as a decode batch (plan once, fused append + decode
        # per layer), the prompt entries as a prefill batch: two tables over the
        # same pages
        def sub_table(entries):
            ptr = np.concatenate([[0], np.cumsum([table.indptr[e + 1] - table.indptr[e]
                                                  for e in entries])]).astype(np.int32)
            idx = np.concatenate([table.indices[table.indptr[e]:table.indptr[e + 1]]
                                  for e in entries]).astype(np.int32)
            ll = table.last_len[entries].astype(np.int32)
            return [torch.from_numpy(x).to(dev) for x in (ptr, idx, ll)]
        dec_e, pr_e = list(range(nd)), list(range(nd, b))
        dtab, ptab = sub_table(dec_e), sub_table(pr_e)
        pqo = torch.from_numpy((np.concatenate([[0], np.cumsum(nrows[nd:])]) ).astype(
            np.int32)).to(dev)
        ws = torch.empty(max(pkv.workspace_size(pkv.cache_desc(cache), hq, nd, dmaxp, 0), 256),
                         dtype=torch.uint8, device=dev)

    def step():
        if split:
            plan = pkv.plan(cache, hq, *dtab, dmaxp, workspace=ws)
            for layer in range(nl):
                pkv.run(cache, layer, Q[layer][:nd], plan, spec.sm_scale,
                        k_new=KN[layer][:nd], v_new=VN[layer][:nd], out=out[layer][:nd],
                        lse=lse[layer][:nd])
                pkv.prefill(cache, layer, Q[layer][nd:], pqo, *ptab, spec.sm_scale, pr,
                            k_new=KN[layer][nd:], v_new=VN[layer][nd:], out=out[layer][nd:],
                            lse=lse[layer][nd:])
            return
        if mixed:
            plan = pkv.plan_mixed(cache, hq, qo, *tabs, rows, dmaxp, workspace=mws)
            for layer in range(nl):
                pkv.mixed_run(cache, layer, Q[layer], *tabs, plan, spec.sm_scale, maxr,
                              k_new=KN[layer], v_new=VN[layer], out=out[layer],
                              lse=lse[layer])
            return
        for layer in range(nl):
            pkv.prefill(cache, layer, Q[layer], qo, *tabs, spec.sm_scale, maxr,
                        k_new=KN[layer], v_new=VN[layer], out=out[layer], lse=lse[layer])

    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            graph.replay()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(args.steps):
            graph.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    step_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    p10, p50, p90 = (float(x) for x in np.percentile(step_ms, [10, 50, 90]))

    # algorithmic work per layer: every row's q.k and p.v over the tokens up to
    # its position; bytes: each entry's K/V once, q and out, the new rows'
    # read and their write into the cache
    pos_count = 0
    for i in range(b):
        n, L = int(nrows[i]), int(lengths[i])
        pos_count += n * (L - n) + n * (n + 1) // 2      # sum over rows of (p + 1)
    flops = 4 * d * hq * pos_count
    kv = int(lengths.sum()) * 2 * hkv * d * 2
    by = kv + 2 * rows * hq * d * 2 + rows * hq * 4 + 4 * rows * hkv * d * 2
    launch_us = step_ms.mean() * 1e3 / nl
    gbs = by / (launch_us * 1e-6) / 1e9
    tflops = flops / (launch_us * 1e-6) / 1e12
    log(f"per layer {launch_us:.2f} us: {gbs:.0f} GB/s algorithmic, {tflops:.1f} TFLOP/s")

    result = {
        "metric": "paged prefill / mixed step: achieved HBM GB/s and TFLOP/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"qwen3_4b_like_mixed_{nd}dec_{npr}x{pr}prompt_36l",
                   "entries": b, "rows": rows, "layers": nl, "num_qo_heads": hq,
                   "num_kv_heads": hkv, "head_dim": d, "page_size": ps,
                   "call": ("pkv_plan + per layer pkv_run (decode entries) and pkv_prefill "
                            "(prompt entries)") if split else
                           ("pkv_plan_mixed + per layer pkv_mixed_run over all entries"
                            if mixed else "pkv_prefill over all entries"),
                   "hip_graph": True},
        "ms_per_step_p10_median_p90": [round(p10, 5), round(p50, 5), round(p90, 5)],
        # with decode rows the step streams their K/V (HBM-bound); prompts
        # alone are a dense contraction, priced against the bf16 MFMA peak
        "roofline": {"bound": "hbm" if nd > 0 else "mfma",
                     "kernel": ("run_kernel + prefill_kernel" if split or mixed
                                else "prefill_kernel"),
                     "achieved": round(gbs, 1) if nd > 0 else round(tflops, 2),
                     "peak": HBM_PEAK_GBS if nd > 0 else MFMA_BF16_PEAK_TFLOPS,
                     "unit": "GB/s" if nd > 0 else "TFLOP/s",
                     "frac": round(gbs / HBM_PEAK_GBS if nd > 0
                                   else tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "hbm_gbs": round(gbs, 1), "bytes_per_launch": by,
                     "avg_launch_us": round(launch_us, 3),
                     "flops_per_launch": flops, "tflops": round(tflops, 2),
                     "mfma_bf16_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                     "timing": "HIP events between graph replays of the 36-layer step; "
                               "per layer = step / 36 (all launches of the layer)"},
    }
    if not args.no_check:
        # sampled rows of layer 0 against the oracle: two decode rows, the
        # first, middle and last rows of one prompt
        import oracle
        ent = [0, 1, nd] if nd > 1 else [nd]
        picks = ([(0, 0), (1, 0)] if nd > 1 else []) + [(nd, 0), (nd, pr // 2), (nd, pr - 1)]
        mini, ip, ix, ll = _host_entries(table, cache[0], ent, torch)
        qsub = np.concatenate([[0], np.cumsum([nrows[e] for e in ent])]).astype(np.int32)
        qh = np.concatenate([_u16(Q[0])[qo_h[e]:qo_h[e + 1]] for e in ent])
        ro, rl = oracle.prefill(mini, 0, qh, qsub, ip, ix, ll, spec.sm_scale)
        got, ref, lg, lr = [], [], [], []
        for e, j in picks:
            k = ent.index(e)
            r_g, r_s = qo_h[e] + j, qsub[k] + j
            got.append(workloads.bf16_to_f32(_u16(out[0, r_g])).astype(np.float64))
            ref.append(ro[r_s])
            lg.append(lse[0, r_g].cpu().numpy().astype(np.float64))
            lr.append(rl[r_s])
        worst = prefill_parity(np.stack(got), np.stack(ref), np.stack(lg), np.stack(lr))
        worst["rows"] = len(picks) * hq
        result["parity"] = worst
        log(f"parity on sampled rows: {worst}")
    if not args.no_cpu_baseline:
        import oracle
        ent = [0, nd] if nd > 0 else [0]
        mini, ip, ix, ll = _host_entries(table, cache[0], ent, torch)
        qsub = np.concatenate([[0], np.cumsum([nrows[e] for e in ent])]).astype(np.int32)
        qh = np.concatenate([_u16(Q[0])[qo_h[e]:qo_h[e + 1]] for e in ent])
        t = time.perf_counter()
        oracle.prefill(mini, 0, qh, qsub, ip, ix, ll, spec.sm_scale)
        dt = time.perf_counter() - t
        f_s = 4 * d * hq * sum(int(nrows[e]) * (int(lengths[e]) - int(nrows[e]))
                               + int(nrows[e]) * (int(nrows[e]) + 1) // 2 for e in ent)
        result["cpu_baseline"] = {"value": round(f_s / dt / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"layer 0, one decode row and one {pr}-row "
                                            f"prompt, {dt:.2f} s"}
    print(json.dumps(result), flush=True)
    return 0


def prefill_parity(got, ref, lse_got, lse_ref):
    """The paged prefill's parity bars (the same as its GPU tests): every
    output element within half a bf16 step of the fp64 value plus 1e-3, the
    mean error within 2^-8 of the mean |output| plus 1e-4, lse within 1e-3."""
    err = np.abs(got - ref)
    res = {"out_max": float(err.max()), "out_mean": float(err.mean()),
           "lse_max": float(np.abs(lse_got - lse_ref).max())}
    res["pass"] = bool(np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-3)
                       and res["out_mean"] <= 2.0 ** -8 * float(np.abs(ref).mean()) + 1e-4
                       and res["lse_max"] <= 1e-3)
    return res


def _host_entries(table, cache_layer, entries, torch):
    """Compact host copy of some entries' pages (ids renumbered from 1)."""
    pages = [table.indices[table.indptr[e]:table.indptr[e + 1]] for e in entries]
    flat = np.concatenate(pages).astype(np.int64)
    hp = cache_layer[torch.from_numpy(flat).to(cache_layer.device)]
    hp = hp.view(torch.int16).cpu().numpy().view(np.uint16)
    mini = np.zeros((1, 1 + len(flat)) + hp.shape[1:], dtype=np.uint16)
    mini[0, 1:] = hp
    indptr = np.concatenate([[0], np.cumsum([len(p) for p in pages])]).astype(np.int32)
    indices = np.arange(1, 1 + len(flat), dtype=np.int32)
    last = np.asarray(table.last_len)[list(entries)].astype(np.int32)
    return mini, indptr, indices, last


def _u16(t):
    return t.contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16)


def check_sample(spec, table, cache, Q, KN, VN, out, lse, torch, nr=None):
    """Sampled rows of the benchmarked step against the oracle (layers 0, mid, last).

    The timed steps re-append the same rows, so the cache now holds the
    post-append state; the oracle appends again (a no-op on those bytes) from
    the same k_new / v_new.  With the fused q/k norm + rotary step (``nr``)
    the oracle runs that step on the sampled entries instead and decodes its
    own bf16-rounded q."""
    import oracle
    from workloads import bf16_to_f32
    act = np.flatnonzero(table.active)
    order = act[np.argsort(table.lengths[act])]
    entries = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    heads = [0, spec.num_qo_heads // 2, spec.num_qo_heads - 1]
    worst = {"out_max": 0.0, "out_mean": 0.0, "lse_max": 0.0, "rows": 0}
    for layer in sorted({0, spec.num_layers // 2, spec.num_layers - 1}):
        mini, ip, ix, ll = _host_entries(table, cache[layer], entries, torch)
        q_rows = _u16(Q[layer])[entries]
        if nr is None:
            oracle.append(mini, 0, _u16(KN[layer])[entries], _u16(VN[layer])[entries], ip,
                          ix, ll)
        elif "axis" in nr:
            q_ref, _ = oracle.qk_norm_mrope_append(
                mini, 0, q_rows, _u16(KN[layer])[entries], _u16(VN[layer])[entries],
                _u16(nr["qw"][layer]), _u16(nr["kw"][layer]), nr["eps"], nr["theta"],
                nr["pos3"].cpu().numpy()[entries], nr["axis"], ip, ix, ll)
            q_rows = oracle.bf16_round(q_ref)
        else:
            q_ref, _ = oracle.qk_norm_rope_append(
                mini, 0, q_rows, _u16(KN[layer])[entries], _u16(VN[layer])[entries],
                _u16(nr["qw"][layer]), _u16(nr["kw"][layer]), nr["eps"], nr["theta"],
                nr["pos"].cpu().numpy()[entries], ip, ix, ll)
            q_rows = oracle.bf16_round(q_ref)
        rb = np.repeat(np.arange(len(entries)), len(heads))
        rh = np.tile(heads, len(entries))
        ro, rl = oracle.decode_rows(mini, 0, q_rows, ip, ix, ll, spec.sm_scale, rb, rh)
        eb = np.asarray(entries)[rb]
        og = bf16_to_f32(_u16(out[layer])[eb, rh]).astype(np.float64)
        lg = lse[layer].cpu().numpy()[eb, rh].astype(np.float64)
        e = np.abs(og - ro)
        worst["out_max"] = max(worst["out_max"], float(e.max()))
        worst["out_mean"] = max(worst["out_mean"], float(e.mean()))
        worst["lse_max"] = max(worst["lse_max"], float(np.abs(lg - rl).max()))
        worst["rows"] += len(rb)
    worst["pass"] = bool(worst["out_max"] <= 1e-2 and worst["out_mean"] <= 1e-3
                         and worst["lse_max"] <= 1e-3)
    return worst


def norm_rope_oracle_time(table, Q, KN, VN, nr, nbytes):
    """The oracle's fused q/k norm + rotary + KV write on layer 0's whole batch
    (one thread), into a host copy of just the pages it writes."""
    import oracle
    b = table.batch
    last = table.indices[table.indptr[1:] - 1]
    pages, inv = np.unique(last, return_inverse=True)
    hkv, d = KN.shape[2], KN.shape[3]
    mini = np.zeros((1, len(pages), 2, table.page_size, hkv, d), dtype=np.uint16)
    ip = np.arange(b + 1, dtype=np.int32)
    ix = inv.astype(np.int32)
    q, kn, vn = _u16(Q[0]), _u16(KN[0]), _u16(VN[0])
    qw, kw = _u16(nr["qw"][0]), _u16(nr["kw"][0])
    pos = nr["pos"].cpu().numpy()
    t = time.perf_counter()
    reps = 0
    while True:
        if "axis" in nr:
            oracle.qk_norm_mrope_append(mini, 0, q, kn, vn, qw, kw, nr["eps"], nr["theta"],
                                        nr["pos3"].cpu().numpy(), nr["axis"], ip, ix,
                                        table.last_len)
        else:
            oracle.qk_norm_rope_append(mini, 0, q, kn, vn, qw, kw, nr["eps"], nr["theta"],
                                       pos, ip, ix, table.last_len)
        reps += 1
        dt = time.perf_counter() - t
        if dt > 1.0:
            break
    return {"us_per_launch": round(dt / reps * 1e6, 1), "cores": 1, "kind": "oracle",
            "gbs": round(nbytes / (dt / reps) / 1e9, 3),
            "sample": f"layer 0, all {b} entries, {reps} calls"}


def host_cpus():
    """The host CPUs this process may run on: every CPU of its affinity set,
    within the cgroup CPU quota when one is set, and what /proc/cpuinfo says
    about them (model name, family / model / stepping, logical CPUs)."""
    aff = len(os.sched_getaffinity(0))
    quota = None
    for path in ("/sys/fs/cgroup/cpu.max", "/sys/fs/cgroup/cpu/cpu.cfs_quota_us"):
        try:
            txt = open(path).read().split()
        except OSError:
            continue
        if path.endswith("cpu.max") and txt and txt[0] != "max":
            quota = int(txt[0]) / int(txt[1])
        elif path.endswith("cfs_quota_us") and txt and int(txt[0]) > 0:
            period = int(open("/sys/fs/cgroup/cpu/cpu.cfs_period_us").read())
            quota = int(txt[0]) / period
        break
    threads = aff if quota is None else max(1, min(aff, math.ceil(quota)))
    info = {"model": "", "family": "", "model_id": "", "stepping": "", "logical_cpus": 0}
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k == "processor":
                info["logical_cpus"] += 1
            elif k == "model name" and not info["model"]:
                info["model"] = v
            elif k == "cpu family" and not info["family"]:
                info["family"] = v
            elif k == "model" and not info["model_id"]:
                info["model_id"] = v
            elif k == "stepping" and not info["stepping"]:
                info["stepping"] = v
    except OSError:
        pass
    info.update({"threads": threads, "affinity_cpus": aff, "nproc": os.cpu_count(),
                 "cgroup_cpu_quota": quota})
    return info


def cpu_baseline(spec, table, cache, Q, KN, VN, torch, seconds):
    """The fp64 oracle (as it stands) on a bounded sample of the workload.

    Sample: whole layers of the step, in order, every query head of every
    active entry, until about ``seconds`` of CPU time (summed over the worker
    threads) have been spent or the step's layers run out; the entries of a
    layer run concurrently on a thread pool (the oracle releases the GIL).
    Only the oracle calls are timed, not the copies of the pages to the host.
    The rate uses the same algorithmic-byte formula as the GPU figure.  The
    first layer is then run again on one thread for the single-core rate."""
    import oracle
    hq, hkv, d = spec.num_qo_heads, spec.num_kv_heads, spec.head_dim
    hostcpu = host_cpus()
    threads = hostcpu["threads"]
    act = [int(e) for e in np.flatnonzero(table.active)]

    def run(job):
        mini, ip, ix, ll, q, k, v = job
        oracle.append(mini, 0, k, v, ip, ix, ll)
        oracle.decode(mini, 0, q, ip, ix, ll, spec.sm_scale)

    dt, layers, nbytes = 0.0, 0, 0
    lens = table.lengths[act]
    per_layer = (int(lens.sum()) * 2 * hkv * d * 2 + len(act) * hq * d * 2 * 2
                 + len(act) * hq * 4 + len(act) * 2 * 2 * hkv * d * 2)
    def layer_jobs(layer):
        qh, kn, vn = _u16(Q[layer]), _u16(KN[layer]), _u16(VN[layer])
        jobs = []
        for e in act:
            mini, ip, ix, ll = _host_entries(table, cache[layer], [e], torch)
            jobs.append((mini, ip, ix, ll, qh[[e]], kn[[e]], vn[[e]]))
        return jobs

    for layer in range(spec.num_layers):
        if dt * threads >= seconds:
            break
        jobs = layer_jobs(layer)
        t = time.perf_counter()
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, jobs))
        dt += time.perf_counter() - t
        layers += 1
        nbytes += per_layer
    jobs = layer_jobs(0)
    t = time.perf_counter()
    for job in jobs:
        run(job)
    dt1 = time.perf_counter() - t
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"layers 0-{layers - 1} of {spec.num_layers}, all {hq} query heads of "
                      f"all {len(act)} active entries ({int(lens.sum())} tokens per layer), "
                      f"append + fp64 decode, {dt:.2f} s on {threads} threads",
            "decode_rows_per_s_equiv": round(len(act) * layers / dt / spec.num_layers, 3),
            "value_1thread": round(per_layer / dt1 / 1e9, 4),
            "sample_1thread": f"layer 0 on one thread, {dt1:.2f} s",
            "cpu_model": hostcpu["model"], "host_cpus": hostcpu}


if __name__ == "__main__":
    sys.exit(main())
