#!/usr/bin/env python3
"""Sparse-FFN decode benchmark on one MI355X.

One step = one decode token batch through every layer of the resident FFN stack: per layer the activation
predictor (sffn_predict) and the neuron-aware sparse FFN (sffn_forward / sffn_forward_q4), layer l+1 reading
layer l's output through the library's normalise-on-load option. Steps are replayed from a HIP graph; inputs
x ~ N(0, 1) are fresh per step and already in HBM when the timed region starts. A workload with a prompt (the
70B Q4_0 stack) also times the prompt as one union-mask batch through the stack, reported beside the decode
figure.

Printed: one JSON line with decode tokens/s (value), HBM GB/s on the active weight rows actually read, the
roofline of the dominant kernel, and the CPU oracle timed on this host's cores over a bounded sample. Kernel
durations come from eager steps of the same stack on the timed inputs: each launch of the profiled kernel
writes its own device start and end timestamps into a HIP event pair on its stream (hipExtLaunchKernelGGL).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "sparse-FFN decode tokens/s + achieved HBM GB/s on active weights (1 MI355X)"
KERNEL_NAMES = {0: "predictor h = P1 x", 1: "predictor z = P2 h + c, threshold, mask",
                2: "compaction + W_gate/W_up row gather + activation", 3: "W_downT column gather"}
FUSED_NAMES = {2: "compaction + W_gate/W_up/W_downT row gather + activation (fused)",
               3: "sum of the per-block partials of y"}
FOLDED_NAMES = {2: "predictor z = P2 h + c, threshold + W_gate/W_up/W_downT row gather + activation (folded)",
                3: "sum of the per-block partials of y + mask and id assembly"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", "--config", default="falcon_40b",
                    help="toy_relu | relullama_7b | llama2_13b | falcon_40b | llama2_70b_q4 (or c1..c5)")
    ap.add_argument("--batch", type=int, default=1, help="tokens per decode step (union mask when > 1)")
    ap.add_argument("--act", choices=("relu", "sqrelu", "reglu"), default=None,
                    help="activation instead of the workload's own (same shapes)")
    ap.add_argument("--hot-prefix", action="store_true",
                    help="declare each layer's saturated neurons (stored first) always active: no predictor rows")
    ap.add_argument("--separate-predictor", action="store_true",
                    help="single tokens: predictor and forward as separate calls (no folded predictor stage 2)")
    ap.add_argument("--rank-schedule", choices=("fixed", "adaptive"), default="fixed",
                    help="adaptive: predictor ranks cycle over 0.5, 1, 1.5, 1 times the workload's rank by layer")
    ap.add_argument("--profile-steps", type=int, default=8, help="eager steps per profiled kernel")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--prompt", type=int, default=None,
                    help="prompt tokens timed as one union batch (default: the workload's own, 64 for the 70B)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also", default="llama2_13b",
                    help="comma-separated workloads measured after the headline one at the same batch, steps and "
                         "warm-up (decode only, no CPU sample), reported under 'also'; 'none' for none")
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly instead of replaying a graph")
    ap.add_argument("--copy-only", type=float, default=None, metavar="MIB",
                    help="only copy MIB mebibytes device to device 8 times and exit (the reference transfer that "
                         "scales the rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ("common.h", "rowgather.h", "api.hip", "predict.hip", "forward.hip", "forward_q4.hip", "union.hip",
                  "union_rows.hip", "union_down.hip", "fused.hip", "decode.hip")


def kernel_source_hash() -> str:
    """sha256 over the kernel sources: counter results taken on other sources are not reported."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "activation_sparse_ffn_predictor_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for(workload: str, batch: int, kernel: str, launches: float):
    """(HBM bytes per launch, detail) of `kernel` measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, each
    scaled by the same counter on a plain copy of known size), if such a measurement exists for these kernel
    sources; None otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    e = t.get("runs", {}).get(f"{workload}/B{batch}", {}).get(kernel)
    if not e:
        return None
    return e["fetch_bytes"] + e["write_bytes"], {
        "fetch_bytes": e["fetch_bytes"], "write_bytes": e["write_bytes"],
        "algorithmic_bytes_per_launch": round(launches, 1), "source": "profiles/traffic.json"}


def copy_only(mib: float):
    import torch
    n = int(mib * 1024 * 1024) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(8):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 4 * n, "launches": 8}), flush=True)


def cpu_baseline(wl, B: int, budget_s: float):
    """The oracle (plain fp64 NumPy dense FFN + predictor) timed on this host over a bounded sample of the same
    workload: whole layers, B tokens per evaluation, until the time budget is spent; extrapolated to the stack.
    BLAS runs on every core of this process's affinity mask; a shorter second sample runs on one thread."""
    import numpy as np
    import oracle
    import synthgen as sg
    cores = len(os.sched_getaffinity(0))
    layers = [0, 1] if wl.L > 1 else [0]
    ws = [oracle.logical_weights(sg.layer_host(wl, l)) for l in layers]
    t_start = time.perf_counter()

    def sample(seconds):
        times, n, step = [], 0, 0
        t0s = time.perf_counter()
        while time.perf_counter() - t0s < seconds:
            for w in ws:
                x = sg.inputs(wl, step, B)
                t0 = time.perf_counter()
                oracle.layer(wl.act, x, w, wl.t)
                times.append(time.perf_counter() - t0)
                n += 1
            step += 1
        return float(np.median(times)), n

    blas_threads, one = None, None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        with threadpool_limits(limits=cores):
            blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
            per_layer, n = sample(budget_s)
        with threadpool_limits(limits=1):               # the same oracle on one BLAS thread, a shorter sample
            one, _ = sample(budget_s / 3.0)
    except ImportError:
        per_layer, n = sample(budget_s)
    tok_s = B / (per_layer * wl.L)
    return {"value": round(tok_s, 4), "unit": "tokens/s", "cores": int(blas_threads or cores), "kind": "oracle",
            "sample": f"{n} layer evaluations of {wl.name} (layers {layers}, {B} token(s) each, fp64 NumPy dense FFN "
                      f"+ predictor), median {per_layer * 1e3:.1f} ms per layer, extrapolated to {wl.L} layers",
            "affinity_cores": cores, "blas_threads": blas_threads,
            "value_1_thread": None if one is None else round(B / (one * wl.L), 4),
            "cpu_model": _cpu_model(),
            "seconds": round(time.perf_counter() - t_start, 2)}


def _cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: model name, family / model / stepping, logical CPUs."""
    info, ncpu = {}, 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "processor":
                    ncpu += 1
                elif k in ("model name", "cpu family", "model", "stepping", "vendor_id") and k not in info:
                    info[k] = v
    except OSError:
        return "unknown"
    return (f"{info.get('model name', 'unknown')} ({info.get('vendor_id', '?')} family {info.get('cpu family', '?')} "
            f"model {info.get('model', '?')} stepping {info.get('stepping', '?')}, {ncpu} logical CPUs visible)")


def measure(wl, B: int, args, with_prompt: bool):
    """Build the resident stack of ``wl`` and time its decode steps (and, if asked, its prompt); returns the
    fields of the JSON line for this workload."""
    import numpy as np
    import torch

    import synthgen as sg
    from activation_sparse_ffn_predictor_amd import _lib
    from activation_sparse_ffn_predictor_amd.stack import SparseFFNStack

    PB = (wl.prompt if args.prompt is None else args.prompt) if with_prompt else 0
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    stack = SparseFFNStack(wl, dev, max_batch=max(B, PB), hot_prefix=args.hot_prefix,
                           fold_predictor=not args.separate_predictor)
    L = len(stack.layers)
    setup_s = time.perf_counter() - t0
    print(f"# setup: {wl.name}, {L} layers resident, {setup_s:.1f} s", file=sys.stderr, flush=True)

    K, W = args.steps, args.warmup
    X = torch.empty((W + K, B, wl.D), dtype=torch.float32, device=dev)
    for s in range(W + K):
        sg.inputs(wl, s, B, tag=sg.TAG_X_DECODE, out=X[s])
    n_acc = torch.zeros(L, dtype=torch.int64, device=dev)
    # the step's token(s) are taken from X by a step counter on the device, inside the replayed graph, so a
    # step is one graph launch with no host-side copy between steps
    step_idx = torch.zeros(1, dtype=torch.long, device=dev)

    def make_run(nb, acc):
        def body():
            if acc is not None:
                stack.x_in[:nb].copy_(X.index_select(0, step_idx)[0])
                step_idx.add_(1)
            stack.step(nb)
            if acc is not None:
                acc.add_(stack.n_active)
        if args.no_graph:
            return body
        body()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        return g.replay

    # ---- optional prompt: PB tokens through the stack as one union-mask batch, timed on its own
    prompt = None
    if PB > 0:
        XP = torch.empty((PB, wl.D), dtype=torch.float32, device=dev)
        sg.inputs(wl, 0, PB, tag=sg.TAG_X_PROMPT, out=XP)
        stack.x_in[:PB].copy_(XP)
        run_p = make_run(PB, None)
        reps = 5
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        for _ in range(2):
            stack.x_in[:PB].copy_(XP)
            run_p()
        torch.cuda.synchronize()
        for i in range(reps):
            stack.x_in[:PB].copy_(XP)
            ev[i].record()
            run_p()
        ev[reps].record()
        torch.cuda.synchronize()
        p_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
        n_p = float(stack.n_active.double().mean().item())
        prompt = {"tokens": PB, "ms_median": round(p_ms[reps // 2], 4), "tokens_s": round(PB / (p_ms[reps // 2] * 1e-3), 1),
                  "union_rows_per_layer": round(n_p, 1), "union_density": round(n_p / wl.F, 4),
                  "active_weight_gbs": round(n_p * stack.active_weight_bytes_per_row() * L / (p_ms[reps // 2] * 1e-3)
                                             / 1e9, 1)}
        print(f"# prompt: {prompt}", file=sys.stderr, flush=True)

    # ---- decode steps: W warm-up replays, then K timed replays with an event between consecutive steps
    run = make_run(B, n_acc)                           # (the capture's eager warm-up step consumed X[0])
    step_idx.zero_()
    for s in range(W):
        run()
    torch.cuda.synchronize()
    n_acc.zero_()
    step_idx.fill_(W)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for s in range(K):
        ev[s].record()
        run()
    ev[K].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = ev[0].elapsed_time(ev[K])
    per_step = np.array([ev[s].elapsed_time(ev[s + 1]) for s in range(K)])
    ms_step = ms_total / K
    n_mean = n_acc.cpu().numpy().astype(np.float64) / K          # mean active rows per layer per step
    row_bytes = stack.active_weight_bytes_per_row()
    active_bytes_step = float(n_mean.sum()) * row_bytes
    pred_bytes_step = stack.predictor_bytes()
    tok_s = B * K / (ms_total * 1e-3)

    # ---- per-kernel durations: P eager steps of the same stack on the timed inputs; every launch of the
    # profiled kernel records its own device start and end timestamps into a HIP event pair on its stream
    P = max(1, args.profile_steps)
    prof, nlog = {}, []
    timing = "eager steps, device timestamps of each launch"
    for kid in (0, 1, 2, 3):
        _lib.profile_begin(kid, P * L)
        for s in range(P):
            stack.x_in[:B].copy_(X[W + (s % K)])
            stack.step(B)
            if kid == 2:
                nlog.append(stack.n_active.cpu().numpy().astype(np.float64))
        prof[kid] = np.asarray(_lib.profile_end(P * L), dtype=np.float64)
    torch.cuda.synchronize()
    prof = {k: v for k, v in prof.items() if len(v)}   # the folded layers launch no separate stage-2 kernel
    mean_us = {k: float(v.mean() * 1e3) for k, v in prof.items()}
    # algorithmic bytes per launch (active rows actually read by the profiled launches)
    n_prof = np.concatenate(nlog) if nlog else np.zeros(1)
    if stack.q4:
        one_row = wl.D // 2 + 2 * (wl.D // 32)
    else:
        one_row = 2 * wl.D
    rows_mats = wl.n_mats - 1
    path = _lib.forward_path(wl.act, stack.q4, B, wl.D, wl.F)
    ranks, hots = np.asarray(stack.ranks, np.float64), np.asarray(stack.n_hot, np.float64)
    fold = np.tile(np.array([stack.folded(i, B) for i in range(L)]), P)   # launches: P steps x L layers
    sep = ~fold
    p2_bytes = np.tile(2.0 * (wl.F - hots) * ranks, P)
    if path == _lib.PATH_FUSED:
        # kernel 2 gathers gate/up and W_downT rows (folded: after reading the block's P2 rows); kernel 3 adds
        # the per-block partial sums of y (folded: all 256 of them, and assembles the mask and ids; fused: those of
        # the max(64, ceil(n / 8)) blocks that took rows, at most n and 256)
        bytes_rows = n_prof * wl.n_mats * one_row + np.where(fold, p2_bytes, 0.0)
        working = np.minimum(np.minimum(np.maximum(64.0, np.ceil(n_prof / 8.0)), 256.0), n_prof)
        bytes_cols = (np.where(fold, 256.0, working) * wl.D + B * wl.D) * 4.0
    else:
        bytes_rows = n_prof * rows_mats * one_row                # per launch of kernel 2
        bytes_cols = n_prof * one_row                            # per launch of kernel 3
    kb = {0: np.tile(2.0 * ranks * wl.D, P), 1: p2_bytes[sep],   # launches in layer order
          2: bytes_rows, 3: bytes_cols}
    tot = {k: float(prof[k].sum()) for k in prof}
    dom = max(tot, key=tot.get)
    m = min(len(kb[dom]), len(prof[dom]))
    achieved = float(kb[dom][:m].sum() / (prof[dom][:m].sum() * 1e-3) / 1e9)       # GB/s
    names = {**KERNEL_NAMES, **(FUSED_NAMES if path == _lib.PATH_FUSED else {}), **(FOLDED_NAMES if fold.all() else {})}
    if fold.any() and not fold.all():
        names[2] += " (folded with the predictor in some layers)"
    fwd_us = mean_us[2] + mean_us[3]
    fwd_gbs = (float(n_prof.mean()) * row_bytes) / (fwd_us * 1e-6) / 1e9

    tr = traffic_for(wl.name, B, names[dom], float(kb[dom][:m].mean()))
    traffic, traffic_detail = tr if tr else (None, None)
    res = {
        "value": round(tok_s, 2),
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_p10_p50_p90": [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)],
        "us_per_layer": round(float(np.median(per_step)) * 1e3 / L, 3),   # FFN-layer time: median step / layers
        "dtype": "f16" if not stack.q4 else "q4_0",
        "config": {"workload": wl.name, "d_model": wl.D, "d_ffn": wl.F,
                   "rank": wl.r if not wl.ranks else list(wl.ranks), "layers": L, "batch": B,
                   "activation": wl.act, "weights": "fp16" if not stack.q4 else "q4_0", "density_target": wl.density,
                   "hot_prefix_per_layer": round(float(np.mean(stack.n_hot)), 1),
                   "predictor_folded_layers": int(fold[:L].sum()), "graph": not args.no_graph},
        "active_weight_gbs": round(active_bytes_step / (ms_step * 1e-3) / 1e9, 1),
        "forward_active_gbs": round(fwd_gbs, 1),
        # the spec quantity: active-weight bytes over the forward kernels' time, against the 8 TB/s peak
        "active_weight_frac": round(fwd_gbs / HBM_PEAK_GBS, 4),
        "all_bytes_gbs": round((active_bytes_step + pred_bytes_step) / (ms_step * 1e-3) / 1e9, 1),
        "active_rows_per_layer": round(float(n_mean.mean()), 1),
        "density": round(float(n_mean.mean()) / wl.F, 4),
        "kernel_us": {names[k]: round(v, 3) for k, v in mean_us.items()},
        "kernel_timing": timing,
        "prompt": prompt,
        # the dominant kernel's algorithmic bytes per launch (the active rows it gathers; for a folded layer its P2
        # rows too; not the partial sums of y, which are this design's overhead), over its own launch time
        "roofline": {"bound": "hbm", "kernel": names[dom], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_detail": traffic_detail},
        "wall_s": round(wall, 3),
        "setup_s": round(setup_s, 1),
    }
    del stack, X, n_acc
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs the sparse-FFN stack on one GPU; --gpus must be 1"}),
              flush=True)
        sys.exit(2)

    if args.copy_only is not None:
        copy_only(args.copy_only)
        return

    import synthgen as sg

    wl = sg.workload(args.workload)
    if args.act and args.act != wl.act:
        wl = sg.custom(wl, act=args.act, name=f"{wl.name}_{args.act}")
    if args.rank_schedule == "adaptive":
        wl = sg.with_rank_schedule(wl)
    B = args.batch
    head = measure(wl, B, args, with_prompt=True)
    also = []
    for name in [a for a in args.also.split(",") if a and a != "none"]:
        other = sg.workload(name)
        if other.name == wl.name:
            continue
        r = measure(other, B, args, with_prompt=False)
        also.append({k: r[k] for k in ("value", "ms_per_step", "us_per_layer", "forward_active_gbs",
                                       "active_weight_frac", "active_weight_gbs", "all_bytes_gbs",
                                       "active_rows_per_layer", "kernel_us", "roofline")}
                    | {"workload": other.name, "batch": B, "unit": "tokens/s"})
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "accumulate": "f32",
        "data": "synthetic",
        **{k: v for k, v in head.items() if k not in ("value", "ms_per_step", "dtype")},
        "also": also,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, B, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
