#!/usr/bin/env python3
"""TT-EmbeddingBag fwd+bwd (fused sparse SGD) benchmark on one MI355X.

A step is one full pass of the hot path over one batch: tt_bag_plan (grouping),
tt_bag_forward_planned, tt_bag_backward_sgd_planned (and tt_cache_lookup first for
the cached workload), all inputs resident in HBM.  Default workload: the README benchmark shape
(p=[200,220,250], q=[4,4,4], ranks=[32,32], E=11,000,000, D=64, 512 bags of 20
uniform indices, SGD lr=0.01) with seeded synthetic data.

Printed (one JSON line): value = microseconds per looked-up index (nnz) of a
whole fwd+bwd step; GFLOPS with 3*(F1+F2) flop per nnz; the roofline of the
dominant kernel (the largest on the step's main stream) from HIP events recorded around
each library launch on its own stream (a separate pass of the same steps); and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
README_US_PER_NNZ = 0.416       # the pages' benchmark line for this workload (hardware unstated)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="readme",
                    choices=["tiny", "readme", "skewed", "multitable", "cached", "readme4"])
    ap.add_argument("--batches", type=int, default=8, help="distinct batches cycled through")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="group each batch right before its forward (no overlap with the "
                         "previous backward)")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per step (plain pipelined path) "
                         "instead of enqueuing each step's calls from the host")
    ap.add_argument("--cache-policy", default="topk", choices=["topk", "lfu32"],
                    help="cached workload: exact top-K or 32-way set-associative LFU")
    ap.add_argument("--update", default="sgd", choices=["sgd", "adagrad", "grad"],
                    help="backward: fused SGD, fused Adagrad (eps 1e-10), or gradients returned")
    ap.add_argument("--dedup", action="store_true",
                    help="backward over distinct indices (tt_bag_plan_dedup + "
                         "tt_bag_backward_*_dedup); no cache, update sgd or grad")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU oracle baseline (0 = skip)")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run device copies of BYTES (counter calibration) and exit")
    return ap.parse_args()


def copy_calibration(nbytes, torch):
    """Plain device-to-device copies of a known size: what FETCH_SIZE / WRITE_SIZE read
    for them turns the counters of the library's kernels into HBM bytes."""
    n = nbytes // 4
    src = torch.rand(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "copies": 5}), flush=True)


def _dev(batch, torch):
    d = {k: torch.from_numpy(batch[k]).cuda() for k in ("indices", "offsets", "grad_out")}
    d["per_sample_weights"] = (torch.from_numpy(batch["per_sample_weights"]).cuda()
                               if batch["per_sample_weights"] is not None else None)
    d["num_bags"] = batch["num_bags"]
    d["np"] = batch
    return d


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    from tensor_train_compressed_ttembeddingbag_amd import abi, metrics, workloads as W
    from tensor_train_compressed_ttembeddingbag_amd.loop import TrainLoop

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, torch)
        return
    abi.lib()
    wl = W.WORKLOADS[args.workload]
    cores = W.make_cores(wl)
    if len(wl.p) != 3:
        run_dcore(args, wl, cores, torch, abi, metrics, W)
        return
    g = [torch.from_numpy(np.concatenate([W.slice_major(cores[t][k]).ravel()
                                          for t in range(wl.num_tables)])).cuda()
         for k in range(3)]
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, wl.num_tables)
    batches = [_dev(W.make_batch(wl, k), torch) for k in range(args.batches)]
    max_nnz = max(b["indices"].numel() for b in batches)
    B = wl.bags_per_table
    cache = rows = slots = aux = aux_rows = None
    csize = 0
    if wl.cache_size:
        policy = abi.TT_CACHE_LFU32 if args.cache_policy == "lfu32" else abi.TT_CACHE_TOPK
        csize = wl.cache_size // 32 * 32 if policy == abi.TT_CACHE_LFU32 else wl.cache_size
        cache = abi.Cache(desc, csize, wl.hashtbl_size, policy=policy)
        for k in range(wl.warmup_batches):
            wb = W.make_batch(wl, 500 + k)
            cache.lookup(torch.from_numpy(wb["indices"]).cuda(), count_freq=True)
        rows = torch.zeros(csize, wl.D, device="cuda")
        torch.cuda.synchronize()
        tp = time.perf_counter()
        n_filled = cache.populate(g, rows)
        populate_ms = (time.perf_counter() - tp) * 1e3
        slots = [torch.empty(b["indices"].numel(), dtype=torch.int32, device="cuda") for b in batches]
    if args.update == "adagrad":  # running sums of squared gradients, from zero
        aux = [torch.zeros_like(x) for x in g]
        aux_rows = torch.zeros_like(rows) if cache is not None else None
    elif args.update == "grad":  # gradient outputs
        aux = [torch.empty_like(x) for x in g]
        aux_rows = torch.empty_like(rows) if cache is not None else None
    # Training loop (loop.TrainLoop): every batch grouped, then the planned forward and
    # backward; by default the grouping of batch i+1 overlaps the backward of batch i.
    pipeline = not args.no_pipeline
    if args.dedup and (cache is not None or args.update == "adagrad"):
        print("--dedup takes no cache and updates by sgd or grad", file=sys.stderr)
        sys.exit(2)
    out = torch.empty(wl.num_tables * B, wl.D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    # --graph: the plain pipelined path replays one captured HIP graph per step
    use_graph = args.graph and pipeline and cache is None and not args.dedup
    loop = TrainLoop(desc, g, batches, B, wl.lr, out, status, update=args.update, aux=aux,
                     aux_rows=aux_rows, cache=cache, rows=rows, slots=slots, dedup=args.dedup,
                     pipeline=pipeline, graph=use_graph)

    def step(_):
        return loop.step()

    def make_eager_step():
        """Per-kernel timing needs the library's own launches (a replayed graph records no
        per-kernel events): the same steps enqueued from the host, on a loop of its own."""
        if not use_graph:
            return step
        le = TrainLoop(desc, g, batches, B, wl.lr, out, status, update=args.update, aux=aux,
                       aux_rows=aux_rows, pipeline=pipeline)
        return lambda _: le.step()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    loop.wait_s = 0.0
    t0 = time.perf_counter()
    done = [step(i) for i in range(args.steps)]
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if int(status.item()) != 0:
        print("device status %d during the benchmark" % int(status.item()), file=sys.stderr)
        sys.exit(1)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    nnz_mean = float(np.mean([batches[i % len(batches)]["indices"].numel() for i in done]))
    us_per_nnz = ms_per_step * 1e3 / nnz_mean
    f1, f2 = metrics.stage_flops(wl.q, wl.ranks)
    step_flops = metrics.step_flops_per_nnz(wl.q, wl.ranks) * nnz_mean
    gflops = step_flops / (ms_per_step * 1e-3) / 1e9

    res = {
        "metric": "TT-EmbeddingBag fwd+bwd µs/nnz and GFLOPS (E=11M, D=64, R=32, B=512)",
        "value": round(us_per_nnz, 6),
        "unit": "us/nnz",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": (round(us_per_nnz / README_US_PER_NNZ, 6) if args.workload == "readme" else None),
        "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64; random-normal cores)",
        "gflops": round(gflops, 3),
        "gflops_convention": "3*(F1+F2)=%d flop per nnz per fwd+bwd step" % (3 * (f1 + f2)),
        "config": {"workload": "%s: p=%s q=%s ranks=%s E=%d D=%d tables=%d bags/table=%d "
                               "nnz/step=%.0f lengths=%s indices=%s weighted=%s lr=%g cache=%d"
                               % (wl.name, list(wl.p), list(wl.q), list(wl.ranks), wl.E, wl.D,
                                  wl.num_tables, B, nnz_mean, list(wl.lengths), list(wl.dist),
                                  wl.weighted, wl.lr, csize),
                   "nnz": nnz_mean, "global_batch": wl.num_tables * B,
                   "update": args.update + (" (backward over distinct indices)"
                                            if args.dedup else ""),
                   "host_enqueue_us_per_step": round((t_enq - t0) * 1e6 / args.steps, 2),
                   # of which waiting for groupings (the rest is the host's own work)
                   "host_wait_us_per_step": round(loop.wait_s * 1e6 / args.steps, 2),
                   "pipeline": ("grouping of batch i+%d beside the backward of batch i"
                                % loop.ahead) if pipeline else "none",
                   "graph": ("one captured HIP graph per step (%d graphs, one per (batch, "
                             "workspace) pair), replayed" % len(loop.graphs))
                            if use_graph else "none"},
    }
    # gradient with respect to the per-sample weights of one planned batch (off the
    # default training step)
    b0 = batches[0]
    wsw = abi.workspace(desc, max_nnz, B, csize)
    cv0 = None
    if cache is not None:
        cv0 = (slots[0], rows)
    if not (wl.D > 512):
        abi.tt_bag_plan(desc, b0["indices"], b0["offsets"], B, b0["per_sample_weights"], cache=cv0,
                        ws=wsw)
        gw = abi.tt_bag_weight_grad(desc, g, b0["indices"], b0["offsets"], B, b0["grad_out"],
                                    b0["per_sample_weights"], cache=cv0, ws=wsw, planned=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(20):
            abi.tt_bag_weight_grad(desc, g, b0["indices"], b0["offsets"], B, b0["grad_out"],
                                   b0["per_sample_weights"], cache=cv0, ws=wsw, out=gw,
                                   planned=True)
        e1.record()
        torch.cuda.synchronize()
        res["config"]["weight_grad_us"] = round(e0.elapsed_time(e1) * 1e3 / 20, 2)
    del wsw
    # initialisation of the workload's cores (approx-normal), off the training path
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    scratch = [torch.empty_like(x) for x in g]
    abi.tt_init_cores(desc, scratch, abi.TT_INIT_APPROX_NORMAL, 1.0, 1)
    ev0.record()
    for r in range(20):
        abi.tt_init_cores(desc, scratch, abi.TT_INIT_APPROX_NORMAL, 1.0, r)
    ev1.record()
    torch.cuda.synchronize()
    init_us = ev0.elapsed_time(ev1) * 1e3 / 20
    nel = sum(x.numel() for x in g)
    res["config"]["init_cores_us"] = round(init_us, 2)
    # full-weight expansion of (up to) 1,000,000 rows of table 0, off the training path
    nrow = min(1_000_000, wl.E)
    dense = torch.empty(nrow, wl.D, device="cuda")
    abi.tt_full_weight(desc, g, 0, nrow, out=dense)
    ev0.record()
    for r in range(5):
        abi.tt_full_weight(desc, g, 0, nrow, out=dense)
    ev1.record()
    torch.cuda.synchronize()
    full_us = ev0.elapsed_time(ev1) * 1e3 / 5
    res["config"]["full_weight_rows"] = nrow
    res["config"]["full_weight_us"] = round(full_us, 1)
    res["config"]["full_weight_gbs"] = round(nrow * wl.D * 4 / (full_us * 1e-6) / 1e9, 1)
    del dense
    res["config"]["init_cores_gbs"] = round(nel * 4 / (init_us * 1e-6) / 1e9, 1)
    if cache is not None:
        res["config"]["cache_rows_filled"] = n_filled
        res["config"]["cache_policy"] = args.cache_policy
        res["config"]["populate_ms"] = round(populate_ms, 3)

    res["config"]["step_us_percentiles"] = step_percentiles(step, min(args.steps, 400), torch)
    if not args.no_roofline:
        res["roofline"], res["kernels"] = roofline(args, wl, batches, make_eager_step(), torch,
                                                   abi, metrics, None if cache is None else slots)
        if use_graph:
            res["roofline"]["kernel_timing"] = ("HIP events of the library's launches in a "
                                                "window of the same steps enqueued eagerly "
                                                "(the timed steps replay graphs)")
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(wl, cores, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def step_percentiles(step, n, torch, window=10):
    """p10 / p50 / p90 of the step time in a separate pass of n steps, each sample the mean
    over a window of `window` consecutive steps: an event on the main stream at every
    window boundary (one event per step would add enough host work per step to make the
    loop wait on the host)."""
    main = torch.cuda.current_stream()
    nw = max(1, n // window)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nw + 1)]
    for k in range(nw * window):
        if k % window == 0:
            evs[k // window].record(main)
        step(k)
    evs[nw].record(main)
    torch.cuda.synchronize()
    t = np.array([evs[k].elapsed_time(evs[k + 1]) * 1e3 / window for k in range(nw)])
    return {"p10": round(float(np.percentile(t, 10)), 2),
            "p50": round(float(np.percentile(t, 50)), 2),
            "p90": round(float(np.percentile(t, 90)), 2), "windows": nw, "window_steps": window}


# kernels the pipelined loop runs on its grouping stream (the plan of a later batch and, with a
# cache, its lookup), beside the step's forward and backward
GROUPING_KERNELS = {"k_route_coop", "k_route_a", "k_route_b", "k_route_c", "k_meta",
                    "k_cache_lookup", "k_dd_keys", "k_dd_count", "k_dd_scan", "k_dd_emit",
                    "k_dd_voff", "k_dd_fill64", "k_sort_hist", "k_sort_scan", "k_sort_scatter"}


def dominant_kernel(kernels, pipelined):
    """The largest kernel (total time) on the step's critical path: in the pipelined loop the
    grouping kernels run on a stream of their own beside the step's kernels, so the pick is
    among the main stream's; without a pipeline every kernel is on the path."""
    onpath = [k for k in kernels if not (pipelined and k in GROUPING_KERNELS)] or list(kernels)
    return max(onpath, key=lambda k: kernels[k]["total_ms"])


def roofline(args, wl, batches, step, torch, abi, metrics, slots):
    """Dominant kernel's achieved rate from HIP events around each launch."""
    nsteps = min(args.steps, 400)
    abi.tt_profile_enable(True)
    done = [step(i) for i in range(nsteps)]
    torch.cuda.synchronize()
    prof = abi.tt_profile_read()
    abi.tt_profile_enable(False)
    kernels = {k: {"total_ms": round(v[0], 4), "launches": v[1],
                   "avg_us": round(1e3 * v[0] / v[1], 3) if v[1] else None}
               for k, v in prof.items() if v[1]}
    dom = dominant_kernel(kernels, not args.no_pipeline)
    # algorithmic work of the contraction kernels, averaged over the batches stepped
    per_batch = []
    for j, b in enumerate(batches):
        nb = b["np"]
        sl = None if slots is None else slots[j].cpu().numpy()
        nel = int(np.sum(sl < 0)) if sl is not None else len(nb["indices"])
        nbw = nel
        if args.dedup:  # the backward runs one element per distinct (table, index)
            tb = (np.searchsorted(nb["offsets"], np.arange(len(nb["indices"])), side="right")
                  - 1) // wl.bags_per_table
            nbw = len(np.unique(tb.astype(np.int64) * wl.E + nb["indices"]))
        per_batch.append((metrics.unique_pairs(wl.p, wl.num_tables, wl.bags_per_table,
                                               nb["indices"], nb["offsets"], sl, wl.E), nel,
                          nbw))
    U = float(np.mean([per_batch[i % len(batches)][0] for i in done]))
    N = float(np.mean([per_batch[i % len(batches)][1] for i in done]))
    Nb = float(np.mean([per_batch[i % len(batches)][2] for i in done]))
    work = {"k_bwd": metrics.bwd_kernel_flops(wl.q, wl.ranks, Nb, U),
            "k_fwd": metrics.fwd_kernel_flops(wl.q, wl.ranks, N, U)}
    avg_s = kernels[dom]["avg_us"] * 1e-6
    from tensor_train_compressed_ttembeddingbag_amd import profiling
    traffic = profiling.read_traffic(
        os.path.join(ROOT, "profiles", "%s_%s_traffic.txt" % (dom, args.workload)), dom)
    if dom in work:
        ach = work[dom] / avg_s / 1e12
        rf = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 3),
              "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
              "frac": round(ach / PEAK_FP32_MFMA_TFLOPS, 4),
              "traffic": None if traffic is None else round(traffic),
              "work_per_launch": "%.4g flop (2*F1 per distinct (i1,i2) pair x %.1f pairs + "
                                 "2*F2 per element x %.1f elements)" % (work[dom], U, Nb)
              if dom == "k_bwd" else "%.4g flop (F1 x %.1f pairs + F2 x %.1f elements)"
                                     % (work[dom], U, N)}
    else:
        # grouping / pooling kernels: algorithmic bytes of the whole grouping step
        NZ = float(np.mean([batches[i % len(batches)]["indices"].numel() for i in done]))
        nbytes = metrics.route_bytes(NZ, wl.num_tables * wl.bags_per_table, wl.weighted,
                                     slots is not None)
        ach = nbytes / avg_s / 1e9
        rf = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 3), "peak": PEAK_HBM_GBS,
              "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 6),
              "traffic": None if traffic is None else round(traffic),
              "work_per_launch": "%.4g bytes (grouping of %.0f elements)" % (nbytes, NZ)}
    for k in ("k_fwd", "k_bwd"):
        if k in kernels:
            kernels[k]["tflops"] = round(work[k] / (kernels[k]["avg_us"] * 1e-6) / 1e12, 3)
    return rf, kernels


def run_dcore(args, wl, cores, torch, abi, metrics, W):
    """d-core workload: a step is tt_bag_plan_d (grouping) + tt_bag_forward_d_planned +
    tt_bag_backward_sgd_d_planned (both multiply out the groups of cores; the backward
    splits the gradients back and applies SGD to the d cores), in the same pipelined loop
    as the three-core workloads (loop.TrainLoop)."""
    from tensor_train_compressed_ttembeddingbag_amd.loop import TrainLoop
    d = len(wl.p)
    g = [torch.from_numpy(np.concatenate([W.slice_major(cores[t][k]).ravel()
                                          for t in range(wl.num_tables)])).cuda()
         for k in range(d)]
    desc = abi.make_desc_d(wl.p, wl.q, wl.ranks, wl.E, wl.num_tables)
    a, b = abi.tt_bag_groups_d(desc)
    q3 = (int(np.prod(wl.q[:a])), int(np.prod(wl.q[a:b])), int(np.prod(wl.q[b:])))
    r3 = (wl.ranks[a - 1], wl.ranks[b - 1])
    batches = [_dev(W.make_batch(wl, k), torch) for k in range(args.batches)]
    B = wl.bags_per_table
    out = torch.empty(wl.num_tables * B, wl.D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    loop = TrainLoop(desc, g, batches, B, wl.lr, out, status, pipeline=not args.no_pipeline)

    def step(_):
        return loop.step()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    done = [step(i) for i in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if int(status.item()) != 0:
        print("device status %d during the benchmark" % int(status.item()), file=sys.stderr)
        sys.exit(1)
    ms = (t1 - t0) * 1e3 / args.steps
    nnz = float(np.mean([batches[i % len(batches)]["indices"].numel() for i in done]))
    res = {"metric": "TT-EmbeddingBag fwd+bwd µs/nnz and GFLOPS (E=11M, D=64, R=32, B=512)",
           "value": round(ms * 1e3 / nnz, 6), "unit": "us/nnz", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded numpy PCG64; random-normal cores)",
           "config": {"workload": "%s: d=%d p=%s q=%s ranks=%s E=%d D=%d tables=%d bags/table=%d "
                                  "cut=[0,%d)[%d,%d)[%d,%d) (as three cores q=%s ranks=%s)"
                      % (wl.name, d, list(wl.p), list(wl.q), list(wl.ranks), wl.E, wl.D,
                         wl.num_tables, B, a, a, b, b, d, list(q3), list(r3)),
                      "nnz": nnz, "global_batch": B, "update": "sgd",
                      "pipeline": "grouping of batch i+1 beside the backward of batch i; the "
                                  "host waits for it before the forward of batch i+1"
                                  if not args.no_pipeline else "none"}}
    res["config"]["step_us_percentiles"] = step_percentiles(step, min(args.steps, 400), torch)
    if not args.no_roofline:
        abi.tt_profile_enable(True)
        done = [step(i) for i in range(min(args.steps, 200))]
        torch.cuda.synchronize()
        prof = abi.tt_profile_read()
        abi.tt_profile_enable(False)
        kernels = {k: {"total_ms": round(v[0], 4), "launches": v[1],
                       "avg_us": round(1e3 * v[0] / v[1], 3)} for k, v in prof.items() if v[1]}
        dom = dominant_kernel(kernels, not args.no_pipeline)
        # the contraction kernels run the three-core shape of the cut
        p3 = (int(np.prod(wl.p[:a])), int(np.prod(wl.p[a:b])), int(np.prod(wl.p[b:])))
        U = float(np.mean([metrics.unique_pairs(p3, wl.num_tables, B, batches[i % len(batches)]["np"]["indices"],
                                                batches[i % len(batches)]["np"]["offsets"], None, wl.E)
                           for i in range(len(batches))]))
        work = {"k_bwd": metrics.bwd_kernel_flops(q3, r3, nnz, U),
                "k_fwd": metrics.fwd_kernel_flops(q3, r3, nnz, U)}
        if dom in work:
            ach = work[dom] / (kernels[dom]["avg_us"] * 1e-6) / 1e12
            res["roofline"] = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 3),
                               "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(ach / PEAK_FP32_MFMA_TFLOPS, 4), "traffic": None,
                               "work_per_launch": "%.4g flop" % work[dom]}
        res["kernels"] = kernels
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(wl, cores, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _host_threads():
    """Cores this process may run on (its affinity mask), capped by OMP_NUM_THREADS when
    the environment sets it (a shared host hands each job a share of its CPUs)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def cpu_baseline(wl, cores, budget_s, reps=5):
    """The oracle, as it stands (single-threaded fp64 C, untouched), on the host's cores:
    fwd+bwd of a prefix of the bags of a batch of the same workload, sized so that one run
    takes about budget / (4 reps) on one core.  One core: reps runs on batch 0's prefix,
    median.  All cores (cores = the threads this process may use): each run gives every
    core its own batch's prefix (batches 0 .. cores-1, disjoint bags of the same
    workload) in its own thread, all at once (the oracle's C calls release the GIL), and
    takes the wall time; median of reps runs.  Value = time per nnz of the whole run.
    With several tables the prefix is taken from table 0 (bags are table-major), run as
    a one-table batch with that table's cores."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from tensor_train_compressed_ttembeddingbag_amd import workloads as W
    oracle.build()
    fwd, bwd = ((oracle.forward, oracle.backward) if len(wl.p) == 3
                else (oracle.forward_d, oracle.backward_d))
    cores = cores[:1]
    all_bags = wl.bags_per_table  # table 0's bags

    def run(b, bags):
        off = b["offsets"]
        n = int(off[bags])
        psw = None if b["per_sample_weights"] is None else b["per_sample_weights"][:n]
        fwd(wl.p, wl.q, wl.ranks, wl.E, cores, b["indices"][:n], off[:bags + 1], bags, psw)
        bwd(wl.p, wl.q, wl.ranks, wl.E, cores, b["indices"][:n], off[:bags + 1], bags,
            b["grad_out"][:bags], psw)
        return n

    b0 = W.make_batch(wl, 0)
    bags = min(16, all_bags)
    while True:  # size the prefix: one run >= budget / (4 reps), or the whole table
        t0 = time.perf_counter()
        run(b0, bags)
        dt = time.perf_counter() - t0
        if dt >= budget_s / (4 * reps) or bags == all_bags:
            break
        bags = min(all_bags, bags * 2)
    one = []
    for _ in range(reps):
        t0 = time.perf_counter()
        n = run(b0, bags)
        one.append((time.perf_counter() - t0) * 1e6 / n)
    nt = _host_threads()
    batches = [b0] + [W.make_batch(wl, k) for k in range(1, nt)]
    allc = []
    with ThreadPoolExecutor(max_workers=nt) as ex:
        for _ in range(reps):
            t0 = time.perf_counter()
            nn = sum(ex.map(lambda b: run(b, bags), batches))
            allc.append((time.perf_counter() - t0) * 1e6 / nn)
    med1, medn = float(np.median(one)), float(np.median(allc))
    return {"value": round(medn, 4), "unit": "us/nnz", "cores": nt, "kind": "oracle",
            "value_1core": round(med1, 3), "cores_1core": 1,
            "runs_us_per_nnz": {"1": [round(x, 3) for x in one],
                                str(nt): [round(x, 4) for x in allc]},
            "cpu_model": _cpu_model(),
            "sample": "fwd+bwd of the first %d of %d bags%s of a batch (%d nnz): one core, "
                      "batch 0, median of %d runs; %d cores, batches 0..%d one per thread "
                      "at once (the oracle's C calls release the GIL), wall time per nnz, "
                      "median of %d runs; fp64 C oracle unchanged; host: %s, %d CPUs "
                      "visible, %d usable"
                      % (bags, all_bags,
                         " of table 0 of %d" % wl.num_tables if wl.num_tables > 1 else "",
                         int(b0["offsets"][bags]), reps, nt, nt - 1, reps, _cpu_model(),
                         os.cpu_count() or 0, nt)}


if __name__ == "__main__":
    main()
