#!/usr/bin/env python3
"""Benchmark of the PowerSGD compression step with error feedback on one MI355X.

Workload: ResNet-18 (CIFAR) gradient shapes, 21 compressed matrices + 41 uncompressed
tensors (11,173,962 parameters), rank 2, W = 16 simulated workers held as 16 slices in
HBM, fp32.  One step = one psgd_compress_step over all tensors (EF add, P = M Q, worker
mean, Gram-Schmidt, Q = M^T P, worker mean, decompress, new errors).  Inputs are
synthetic (planted low-rank part + worker noise), drawn on the device before timing.

Four plan variants are timed: "deferred" (PSGD_FLAG_DEFERRED_ERROR: one pass over the
workers' G and E per step; the error buffer holds M_w and the previous step's P Q^T is
subtracted in the next step's pass), "carry" (PSGD_FLAG_CARRY_ERROR_MEAN: the plain error
E'_w is written every step, and the next step's first pass reads only G plus the
carried error mean), "plain" (no cross-step state) and "local" (PSGD_FLAG_LOCAL_Q_ERROR:
each worker's error uses its own Q_w).  `value` is the --primary one.

A second compressor is timed beside it ("rtopk" in the output): rTop-k with error
feedback on the same shapes and W = 16, 1% of each tensor sent, drawn from its top 2%
(psgd_rtopk_step: EF add, top-set selection, random subset from seeded ranks, sparse
lists, new errors, dense mean update; the deferred-zero plan, whose next step zeroes the
sent entries as it reads the errors), and a third ("atomo"): Spectral-ATOMO on the same
shapes and workers with budget s = 2 (psgd_atomo_step: Gram matrices, tridiagonalisation,
eigenvalues, closed-form probabilities, Bernoulli draws from seeded uniforms, inverse
iteration and back-transformation for the sent atoms, their second factors, the mean).

Prints one JSON line:
  value          gradient GB/s = W * numel * 4 bytes / step time (whole job, one GPU)
  pct_hbm_peak   minimal HBM bytes of a step / step time / 8 TB/s
  pct_hbm_peak_kernel_bytes
                 the bytes the variant's kernels must move (Mbar written and read again,
                 a second pass over the workers) / step time / 8 TB/s
  roofline       the longest kernel: algorithmic bytes per launch / its mean duration
                 (HIP events recorded on the launch stream around every launch)
  cpu_baseline   the CPU oracle timed on a bounded sample of the same workload
"""

from __future__ import annotations

import gc
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
METRIC = "PowerSGD step gradient GB/s (ResNet-18 shapes, r=2, W=16) & % HBM peak"
KERNEL_SRC = os.path.join(ROOT, "distributed_sgd_gradient_ef_amd", "csrc", "kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_resnet18_r2_w16.json")
RTOPK_SRC = os.path.join(ROOT, "distributed_sgd_gradient_ef_amd", "csrc", "rtopk.hip")
RTOPK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_rtopk_resnet18_w16.json")
RTOPK_METRIC = "rTop-k step gradient GB/s (ResNet-18 shapes, 1% sent from the top 2%, W=16) & % HBM peak"
ATOMO_METRIC = "Spectral-ATOMO step gradient GB/s (ResNet-18 shapes, budget s=2, W=16)"
ATOMO_SRC = os.path.join(ROOT, "distributed_sgd_gradient_ef_amd", "csrc", "atomo.hip")
ATOMO_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_atomo_resnet18_w16.json")
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32: the vector peak and the dense MFMA peak are both 157.3


def kernel_bytes(plan, dtype_bytes: int, variant: str) -> dict:
    """Algorithmic HBM bytes per launch of each kernel for this plan and variant."""
    s = plan.sizes
    W = s["n_workers"]
    mn, vn = s["matrix_numel"], s["vector_numel"]
    gb = dtype_bytes
    first = {
        # read G_w and E_w on every worker, write Mbar once
        "plain": W * (gb + 4) + 4,
        # read G_w on every worker and the carried error mean once, write Mbar once
        "carry": W * gb + 8,
        # read G_w and E_w, write M_w on every worker, write Mbar once
        "deferred": W * (gb + 8) + 4,
        # as plain
        "local": W * (gb + 4) + 4,
    }[variant]
    return {
        # 1-D tensors: read G_w on every worker, write the mean once
        "k_first": first * mn + (W * gb + 4) * vn,
        # read Mbar once (P and Q are cache-resident)
        "k_q_partial": 4 * mn,
        # read G_w, E_w and write E'_w on every worker, write U once (and the new error
        # mean in carry mode); 1-D tensors: read the mean, write the update
        "k_apply": (W * (gb + 8) + (8 if variant == "carry" else 4)) * mn + 8 * vn,
        # write U once; 1-D tensors: read the mean, write the update
        "k_update": 4 * mn + 8 * vn,
        # local-Q error: read G_w and E_w on every worker for its own Q_w
        "k_qw_partial": W * (gb + 4) * mn,
    }


def rtopk_kernel_bytes(plan, dtype_bytes: int, deferred: bool = True) -> dict:
    """Algorithmic HBM bytes per launch of the streaming rTop-k kernels (the selection
    kernels in between move a few bytes per segment or per candidate)."""
    s = plan.sizes
    W, n = s["n_workers"], s["numel"]
    return {
        # read G_w and E_w, write M_w on every worker (deferred zeros: and read the
        # previous step's sent mask, one bit per element)
        "rk_ef_hist": W * (dtype_bytes + 8) * n + (W * n // 8 if deferred else 0),
        # read M_w, write one mask bit per entry on every worker
        "rk_mark": W * 4 * n + W * n // 8,
        # read the top mask and the ranks of the top set, write the kept mask
        "rk_keep": W * n // 4 + W * 4 * s["top_total"],
        # read the kept mask, write the list positions and the lists
        "rk_emit": W * n // 4 + W * 8 * s["keep_total"],
        # read every worker's kept mask, write U once
        "rk_update": W * n // 8 + 4 * n,
    }


def atomo_kernel_work(plan) -> dict:
    """Algorithmic work per launch of the Spectral-ATOMO kernels: flops of the Gram
    matrices (lower triangle, k (k + 1) L multiply-adds), of the reduction to a band of
    half-bandwidth 16 (the classical count of a symmetric Householder reduction, 4/3 k^3
    per matrix and worker) and of the bulge chasing (about 12 b^2 flops for each of the
    k^2 / (2 b) reflectors, b = 16); HBM bytes of the passes over G."""
    s = plan.sizes
    W = s["n_workers"]
    gram = band = chase = gbytes = 0
    for L in plan.layers:
        if L.compressed:
            k, long = L.k, max(L.rows, L.cols)
            gram += W * 2 * k * (k + 1) // 2 * long
            band += W * 4 * k ** 3 // 3
            chase += W * 6 * 16 * k * k
            gbytes += W * 4 * L.rows * L.cols
    return {"at_gram": ("flops", gram), "at_band": ("flops", band), "at_chase": ("flops", chase),
            "at_factor": ("bytes", gbytes)}


def traffic_for(kernel: str, traffic_file: str = TRAFFIC_FILE, source: str = KERNEL_SRC):
    """Measured HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(traffic_file) as f:
            t = json.load(f)
        with open(source, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k or t.get("kernel_source_sha256") != sha:
        return None
    return k.get("hbm_bytes_per_launch")


def cpu_baseline(wl, seconds: float) -> dict:
    """Time the CPU oracle on whole steps of the same workload (at least one step)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from distributed_sgd_gradient_ef_amd import workloads as WL
    from oracle import powersgd_ef as O

    grads = WL.grads(wl, 0)
    layers = []
    for i, (_, shp) in enumerate(wl.shapes):
        q = WL.q0(wl, i) if WL.is_matrix(shp, wl.rank) else None
        layers.append(O.LayerState(grads[i], np.zeros_like(grads[i]), q))
    steps, t0 = 0, time.perf_counter()
    while True:
        O.compress_layers(layers)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    t_step = el / steps
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    gbytes = wl.workers * wl.numel() * 4 / 1e9
    # the same oracle on one thread, one whole step
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        O.compress_layers(layers)
        t_one = time.perf_counter() - t1
    return {"value": round(gbytes / t_step, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "value_1thread": round(gbytes / t_one, 4),
            "sample": f"{steps} whole step(s) of the same workload (all 21 matrices and 41 tensors, "
                      f"W=16, r=2), numpy float64 oracle, {t_step:.2f} s per step; BLAS threads = cores; "
                      f"value_1thread: one more step on one thread, {t_one:.2f} s"}


def atomo_cpu_baseline(wl, seconds: float) -> dict:
    """Time the Spectral-ATOMO oracle on whole workers of the same workload (every matrix
    and tensor of one worker per round, at least one round), scaled to W workers."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from distributed_sgd_gradient_ef_amd import workloads as WL
    from oracle import atomo as O

    grads = WL.grads(wl, 0)
    rounds, t0 = 0, time.perf_counter()
    while True:
        w = rounds % wl.workers
        for li, g in enumerate(grads):
            if O.is_matrix(g.shape[1:]):
                x = WL.atomo_uniforms(wl, 0, w, li, min(g.shape[1:]))
                O.compress_matrix(g[w].astype(np.float64), wl.atomo_budget, x)
        rounds += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    t_worker = el / rounds
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    gbytes = wl.workers * wl.numel() * 4 / 1e9
    return {"value": round(gbytes / (t_worker * wl.workers), 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rounds} worker(s) of the same workload (all 21 matrices of one worker per round, "
                      f"float64 numpy SVD oracle), {t_worker:.2f} s per worker, scaled to W={wl.workers}; "
                      f"BLAS threads = cores"}


def rtopk_cpu_baseline(wl, seconds: float, workers: int = 2) -> dict:
    """Time the rTop-k oracle on `workers` of the W workers (every tensor of each, rounds
    until `seconds` have passed, at least one) and scale to a whole step of W workers:
    each worker's selection is independent, the mean of the sparse messages is a small
    share of the work."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from distributed_sgd_gradient_ef_amd import workloads as WL
    from oracle import rtopk_ef as O

    tops, keeps = WL.rtopk_counts(wl)
    grads, ranks = [], []
    for li in range(len(wl.shapes)):
        p = WL.planted(wl, li, 0)
        low = None if p is None else p.dense()
        grads.append(np.stack([WL.grad_layer(wl, li, 0, w, low) for w in range(workers)]))
        ranks.append(np.stack([WL.rtopk_ranks(wl, 0, w, li, tops[li]) for w in range(workers)]))
    errors = [np.zeros_like(g) for g in grads]
    rounds, t0 = 0, time.perf_counter()
    while True:
        O.compress_layers(grads, errors, tops, keeps, ranks)
        rounds += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    t_step = el / rounds * wl.workers / workers
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    gbytes = wl.workers * wl.numel() * 4 / 1e9
    return {"value": round(gbytes / t_step, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rounds} round(s) of {workers} of the {wl.workers} workers (all 62 tensors each, 1% sent "
                      f"from the top 2%), numpy oracle (lexsort top set), {el / rounds:.2f} s per round, scaled "
                      f"to a whole step of {wl.workers} workers ({t_step:.1f} s); BLAS threads = cores (the "
                      f"selection itself runs on one thread)"}


def timed_steps(torch, step, steps: int, stream):
    """Run `steps` calls of step() with an event recorded on `stream` between calls.
    Returns (mean ms over the whole region, median ms, minimum ms)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    # no garbage-collection pause while the steps are enqueued: a pause of a few ms with
    # the queue short leaves the GPU idle inside the timed region
    gc_was_on = gc.isenabled()
    gc.disable()
    try:
        ev[0].record(stream)
        for i in range(steps):
            step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
    finally:
        if gc_was_on:
            gc.enable()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[steps]) / steps, per[len(per) // 2], per[0]


def config_timings(torch, psgd, WL, dev, steps: int) -> dict:
    """Context lines for the other configurations (not the metric), deferred mode: the
    single small matrix as latency, the LSTM shapes, the bandwidth-stress set at r = 1, 2,
    4 and with bf16 gradients, and the fused momentum step on the ResNet-18 shapes."""
    out = {}

    def run(name, wl, grads, gbytes, nsteps, momentum=False, dtype=None, graph=False):
        W = wl.workers
        shapes = [s for _, s in wl.shapes]
        plan = psgd.psgd_plan_create(shapes, wl.rank, W, dtype if dtype is not None else psgd.PSGD_F32,
                                     psgd.PSGD_FLAG_DEFERRED_ERROR)
        s = plan.sizes
        ld = s["worker_stride"]
        errors = torch.zeros((W, ld), dtype=torch.float32, device=dev)
        q = torch.zeros(s["q_elems"], dtype=torch.float32, device=dev)
        p = torch.zeros(s["p_elems"], dtype=torch.float32, device=dev)
        update = torch.zeros(ld, dtype=torch.float32, device=dev)
        workspace = torch.empty(s["workspace_bytes"], dtype=torch.uint8, device=dev)
        qh = psgd.pack_factors(plan, {i: WL.q0(wl, i) for i, L in enumerate(plan.layers) if L.compressed}, "q")
        q.copy_(torch.from_numpy(qh).to(dev))
        stream = torch.cuda.current_stream(dev)
        if momentum:
            mom = torch.zeros(ld, dtype=torch.float32, device=dev)
            x = torch.zeros(ld, dtype=torch.float32, device=dev)

            def step():
                psgd.psgd_ef_momentum_apply(plan, grads, errors, q, p, mom, x, wl.lr, wl.mu, None, workspace, stream)
            model = s["model_bytes_momentum"]
        else:
            def step():
                psgd.psgd_compress_step(plan, grads, errors, q, p, update, workspace, stream)
            model = s["model_bytes"]
        for _ in range(3):
            step()
        torch.cuda.synchronize(dev)
        ms, med, mn = timed_steps(torch, step, nsteps, stream)
        out[name] = {"workers": W, "rank": wl.rank, "params": s["numel"], "steps": nsteps,
                     "ms_per_step": round(ms, 4), "ms_median": round(med, 4), "ms_min": round(mn, 4),
                     "grad_GBps": round(W * s["numel"] * gbytes / (ms * 1e-3) / 1e9, 1),
                     "pct_hbm_peak": round(100.0 * model / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 2)}
        if graph:  # the same step captured once into a HIP graph and replayed
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):  # on the capture stream (the current one inside)
                psgd.psgd_compress_step(plan, grads, errors, q, p, update, workspace)
            torch.cuda.synchronize(dev)
            ms_g, _, _ = timed_steps(torch, g.replay, nsteps, stream)
            out[name]["ms_per_step_graph_replay"] = round(ms_g, 4)
            del g
        del errors, q, p, update, workspace, plan

    def draw(wl):
        plan = psgd.psgd_plan_create([s for _, s in wl.shapes], wl.rank, wl.workers)
        g = torch.zeros((wl.workers, plan.sizes["worker_stride"]), dtype=torch.float32, device=dev)
        WL.device_grads(wl, 0, [(L.offset, L.rows, L.cols) for L in plan.layers], g)
        return g

    wl = WL.workload("single")
    run("single", wl, draw(wl), 4, 10 * steps, graph=True)
    out["single"]["role"] = "latency (one 256x128 matrix, W=1, r=1; launch-bound)"
    wl = WL.workload("lstm")
    g = draw(wl)
    run("lstm", wl, g, 4, steps)
    del g
    wl = WL.workload("resnet18_momentum")
    g = draw(wl)
    run("resnet18_momentum", wl, g, 4, steps, momentum=True)
    del g
    wl = WL.workload("stress", rank=2)
    g = draw(wl)
    nstress = max(3, steps // 10)
    for r in (1, 2, 4):
        run(f"stress_r{r}", WL.workload("stress", rank=r), g, 4, nstress)
    gb = g.to(torch.bfloat16)
    del g
    torch.cuda.empty_cache()
    run("stress_r2_bf16", wl, gb, 2, nstress, dtype=psgd.PSGD_BF16)
    del gb
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline sample length")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the context timings of the other configurations")
    ap.add_argument("--mode", choices=["all", "carry", "plain", "deferred", "local", "rtopk", "atomo"], default="all",
                    help="plan variants to time (profiling runs use one); rtopk times only the rTop-k step")
    ap.add_argument("--primary", choices=["carry", "deferred", "plain", "local"], default="deferred",
                    help="variant reported as `value` when several are timed")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the W data-parallel workers are simulated as slices of "
              "one GPU's HBM, and no multi-GPU path is built. Use --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from distributed_sgd_gradient_ef_amd import psgd
    from distributed_sgd_gradient_ef_amd import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    psgd.load_library()
    dev = torch.device("cuda:0")
    wl = WL.workload("resnet18")
    shapes = [s for _, s in wl.shapes]
    W = wl.workers
    flag_of = {"plain": 0, "carry": psgd.PSGD_FLAG_CARRY_ERROR_MEAN, "deferred": psgd.PSGD_FLAG_DEFERRED_ERROR,
               "local": psgd.PSGD_FLAG_LOCAL_Q_ERROR}

    def measure(variant: str) -> dict:
        flags = flag_of[variant]
        plan = psgd.psgd_plan_create(shapes, wl.rank, W, psgd.PSGD_F32, flags)
        s = plan.sizes
        ld = s["worker_stride"]
        grads = torch.zeros((W, ld), dtype=torch.float32, device=dev)
        errors = torch.zeros((W, ld), dtype=torch.float32, device=dev)
        q = torch.zeros(s["q_elems"], dtype=torch.float32, device=dev)
        p = torch.zeros(s["p_elems"], dtype=torch.float32, device=dev)
        update = torch.zeros(ld, dtype=torch.float32, device=dev)
        workspace = torch.empty(s["workspace_bytes"], dtype=torch.uint8, device=dev)
        WL.device_grads(wl, 0, [(L.offset, L.rows, L.cols) for L in plan.layers], grads)
        qh = psgd.pack_factors(plan, {i: WL.q0(wl, i) for i, L in enumerate(plan.layers) if L.compressed}, "q")
        q.copy_(torch.from_numpy(qh).to(dev))
        stream = torch.cuda.current_stream(dev)

        def step():
            psgd.psgd_compress_step(plan, grads, errors, q, p, update, workspace, stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize(dev)
        # timed region 1: the step as a caller runs it (an event between steps)
        ms, ms_med, ms_min = timed_steps(torch, step, args.steps, stream)
        # timed region 2: the same steps with every kernel bracketed by HIP events
        psgd.psgd_plan_set_timing(plan, True)
        psgd.psgd_plan_kernel_stats(plan, reset=True)
        t2, t3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t2.record(stream)
        for _ in range(args.steps):
            step()
        t3.record(stream)
        torch.cuda.synchronize(dev)
        ms_timed = t2.elapsed_time(t3) / args.steps
        stats = psgd.psgd_plan_kernel_stats(plan, reset=True)
        psgd.psgd_plan_set_timing(plan, False)
        # timed region 3 (context): one step captured into a HIP graph, replayed K times
        ms_graph = None
        if variant == args.primary:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                psgd.psgd_compress_step(plan, grads, errors, q, p, update, workspace)
            torch.cuda.synchronize(dev)
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            for _ in range(args.steps):
                graph.replay()
            g1.record(stream)
            torch.cuda.synchronize(dev)
            ms_graph = g0.elapsed_time(g1) / args.steps
            del graph
        kb = kernel_bytes(plan, 4, variant)
        kernels = {}
        for name, (n, tot) in stats.items():
            us = 1e3 * tot / max(n, 1)
            entry = {"mean_us": round(us, 2), "launches": n}
            if name in kb:
                entry["alg_bytes"] = kb[name]
                entry["alg_GBps"] = round(kb[name] / (us * 1e-6) / 1e9, 1)
            kernels[name] = entry
        grad_bytes = W * s["numel"] * 4
        # the variant's own bytes: what its kernels must move per step (reads of Mbar and
        # of a second pass included), beside the minimal-bytes model of the step
        own = sum(kb[k] * n for k, (n, _) in stats.items() if k in kb) / max(args.steps, 1)
        del grads, errors, workspace
        return {"ms": ms, "ms_med": ms_med, "ms_min": ms_min, "ms_timed": ms_timed, "ms_graph": ms_graph,
                "kernels": kernels, "kb": kb, "own_bytes": int(own),
                "pct_own": 100.0 * own / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                "sizes": s,
                "value": grad_bytes / (ms * 1e-3) / 1e9, "grad_bytes": grad_bytes,
                "pct": 100.0 * s["model_bytes"] / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)}

    # context: the plain-copy bandwidth the device reaches (1 GiB read + 1 GiB written)
    cbytes = 1 << 30
    src = torch.empty(cbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    psgd.psgd_stream_copy(src, dst, cbytes)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    c0.record()
    for _ in range(5):
        psgd.psgd_stream_copy(src, dst, cbytes)
    c1.record()
    torch.cuda.synchronize(dev)
    copy_gbs = 2 * cbytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    def measure_rtopk() -> dict:
        wr = WL.workload("resnet18_rtopk")
        tops, keeps = WL.rtopk_counts(wr)
        plan = psgd.psgd_rtopk_plan_create(shapes, tops, keeps, W, psgd.PSGD_F32, psgd.PSGD_RTOPK_FLAG_DEFERRED_ZERO)
        s = plan.sizes
        ld = s["worker_stride"]
        # four gradient sets resident in HBM, one per step in turn, so the error memory
        # evolves as under changing gradients rather than one repeated gradient
        nsets = 4
        grads = torch.zeros((nsets, W, ld), dtype=torch.float32, device=dev)
        errors = torch.zeros((W, ld), dtype=torch.float32, device=dev)
        index = torch.zeros((W, s["keep_total"]), dtype=torch.int32, device=dev)
        value = torch.zeros((W, s["keep_total"]), dtype=torch.float32, device=dev)
        update = torch.zeros(ld, dtype=torch.float32, device=dev)
        workspace = torch.empty(s["workspace_bytes"], dtype=torch.uint8, device=dev)
        layout = [(L.offset, L.rows, L.cols) for L in plan.layers]
        ranks = torch.zeros((nsets, W, s["top_total"]), dtype=torch.int32, device=dev)
        for k in range(nsets):
            WL.device_grads(wr, k, layout, grads[k])
            ranks_h = psgd.pack_rows(plan, [np.stack([WL.rtopk_ranks(wr, k, w, li, tops[li]) for w in range(W)])
                                            for li in range(len(shapes))], "top", np.uint32)
            ranks[k].copy_(torch.from_numpy(ranks_h.view(np.int32)))
        stream = torch.cuda.current_stream(dev)
        turn = [0]

        def step():
            k = turn[0] % nsets
            turn[0] += 1
            psgd.psgd_rtopk_step(plan, grads[k], errors, ranks[k], index, value, update, workspace, stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize(dev)
        ms, ms_med, ms_min = timed_steps(torch, step, args.steps, stream)
        psgd.psgd_rtopk_plan_set_timing(plan, True)
        psgd.psgd_rtopk_plan_kernel_stats(plan, reset=True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize(dev)
        stats = psgd.psgd_rtopk_plan_kernel_stats(plan, reset=True)
        psgd.psgd_rtopk_plan_set_timing(plan, False)
        kb = rtopk_kernel_bytes(plan, 4)
        kernels = {}
        for name, (n, tot) in stats.items():
            us = 1e3 * tot / max(n, 1)
            entry = {"mean_us": round(us, 2), "launches": n}
            if name in kb:
                entry["alg_bytes"] = kb[name]
                entry["alg_GBps"] = round(kb[name] / (us * 1e-6) / 1e9, 1)
            kernels[name] = entry
        dom = max((k for k in kernels if k in kb), key=lambda k: kernels[k]["mean_us"])
        dom_us = kernels[dom]["mean_us"]
        achieved = kb[dom] / (dom_us * 1e-6) / 1e9
        grad_bytes = W * s["numel"] * 4
        del grads, errors, workspace
        return {
            "metric": RTOPK_METRIC,
            "value": round(grad_bytes / (ms * 1e-3) / 1e9, 2),
            "unit": "GB/s",
            "ms_per_step": round(ms, 4),
            "ms_per_step_median": round(ms_med, 4),
            "ms_per_step_min": round(ms_min, 4),
            "pct_hbm_peak": round(100.0 * s["model_bytes"] / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 2),
            "model_bytes_per_step": s["model_bytes"],
            "config": {"workload": "resnet18_cifar_shapes", "workers": W, "tensors": s["n_layers"],
                       "keep_frac": wr.keep_frac, "top_factor": wr.top_factor, "keep_total": s["keep_total"],
                       "top_total": s["top_total"], "grad_bytes_per_step": grad_bytes,
                       "gradient_sets": nsets, "plan_flags": "PSGD_RTOPK_FLAG_DEFERRED_ZERO"},
            "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_for(dom, RTOPK_TRAFFIC_FILE, RTOPK_SRC),
                         "alg_bytes_per_launch": kb[dom], "mean_us": dom_us},
            "kernels": kernels,
            **({} if args.no_cpu_baseline else {"cpu_baseline": rtopk_cpu_baseline(wr, args.cpu_seconds / 3)}),
        }

    def measure_atomo() -> dict:
        wa = WL.workload("resnet18_atomo")
        plan = psgd.psgd_atomo_plan_create(shapes, wa.atomo_budget, W)
        s = plan.sizes
        ld, sv = s["worker_stride"], s["sv_total"]
        nsets = 2
        grads = torch.zeros((nsets, W, ld), dtype=torch.float32, device=dev)
        unif = torch.zeros((nsets, W, sv), dtype=torch.float32, device=dev)
        layout = [(L.offset, L.rows, L.cols) for L in plan.layers]
        for k in range(nsets):
            WL.device_grads(wa, k, layout, grads[k])
            xs = {li: np.stack([WL.atomo_uniforms(wa, k, w, li, L.k) for w in range(W)])
                  for li, L in enumerate(plan.layers) if L.compressed}
            unif[k].copy_(torch.from_numpy(psgd.pack_sv(plan, xs)))
        sigma = torch.zeros((W, sv), dtype=torch.float32, device=dev)
        prob = torch.zeros_like(sigma)
        index = torch.zeros((W, sv), dtype=torch.int32, device=dev)
        count = torch.zeros((W, s["n_matrices"]), dtype=torch.int32, device=dev)
        atoms = torch.zeros((W, s["atom_total"]), dtype=torch.float32, device=dev)
        update = torch.zeros(ld, dtype=torch.float32, device=dev)
        workspace = torch.empty(s["workspace_bytes"], dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream(dev)
        turn = [0]

        def step():
            k = turn[0] % nsets
            turn[0] += 1
            psgd.psgd_atomo_step(plan, grads[k], unif[k], sigma, prob, index, count, atoms, update, workspace,
                                 stream)

        nsteps = max(1, min(args.steps, 20))
        for _ in range(min(args.warmup, 3)):
            step()
        torch.cuda.synchronize(dev)
        ms, ms_med, ms_min = timed_steps(torch, step, nsteps, stream)
        psgd.psgd_atomo_plan_set_timing(plan, True)
        psgd.psgd_atomo_plan_kernel_stats(plan, reset=True)
        for _ in range(nsteps):
            step()
        torch.cuda.synchronize(dev)
        stats = psgd.psgd_atomo_plan_kernel_stats(plan, reset=True)
        psgd.psgd_atomo_plan_set_timing(plan, False)
        sent = float(count.float().mean().item())
        work = atomo_kernel_work(plan)
        kernels = {}
        for name, (n, tot) in stats.items():
            us = 1e3 * tot / max(n, 1)
            entry = {"mean_us": round(us, 2), "launches": n}
            if name in work:
                kind, amount = work[name]
                entry["alg_" + kind] = amount
                if kind == "flops":
                    entry["alg_TFLOPs"] = round(amount / (us * 1e-6) / 1e12, 3)
                else:
                    entry["alg_GBps"] = round(amount / (us * 1e-6) / 1e9, 1)
            kernels[name] = entry
        dom = max(kernels, key=lambda k: kernels[k]["mean_us"])
        dom_us = kernels[dom]["mean_us"]
        kind, amount = work.get(dom, ("flops", 0))
        if kind == "flops":
            achieved = amount / (dom_us * 1e-6) / 1e12
            roof = {"kernel": dom, "bound": "mfma" if dom in ("at_gram", "at_band") else "alu",
                    "achieved": round(achieved, 3), "peak": FP32_VECTOR_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / FP32_VECTOR_PEAK_TFLOPS, 5)}
        else:
            achieved = amount / (dom_us * 1e-6) / 1e9
            roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        roof.update({"traffic": traffic_for(dom, ATOMO_TRAFFIC_FILE, ATOMO_SRC), "alg_" + kind + "_per_launch": amount,
                     "mean_us": dom_us})
        grad_bytes = W * s["numel"] * 4
        del grads, workspace, atoms
        out = {
            "metric": ATOMO_METRIC,
            "value": round(grad_bytes / (ms * 1e-3) / 1e9, 2),
            "unit": "GB/s",
            "ms_per_step": round(ms, 4),
            "ms_per_step_median": round(ms_med, 4),
            "ms_per_step_min": round(ms_min, 4),
            "steps": nsteps,
            "config": {"workload": "resnet18_cifar_shapes", "workers": W, "matrices": s["n_matrices"],
                       "budget": wa.atomo_budget, "sv_total": sv, "grad_bytes_per_step": grad_bytes,
                       "mean_atoms_sent_per_matrix": round(sent, 3), "gradient_sets": nsets},
            "roofline": roof,
            "kernels": kernels,
        }
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = atomo_cpu_baseline(wa, args.cpu_seconds / 3)
        return out

    if args.mode == "atomo":
        out = measure_atomo()
        out.update({"n_gpus": 1, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
                    "vs_baseline": None, "dtype": "f32", "stream_copy_GBps": round(copy_gbs, 1)})
        print(json.dumps(out), flush=True)
        return 0

    if args.mode == "rtopk":
        out = measure_rtopk()
        out.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                    "scaling": "weak", "vs_baseline": None, "dtype": "f32", "stream_copy_GBps": round(copy_gbs, 1)})
        print(json.dumps(out), flush=True)
        return 0

    names = ["plain", "carry", "deferred", "local"] if args.mode == "all" else [args.mode]
    results = {n: measure(n) for n in names}
    primary = args.primary if args.primary in results else names[0]
    main_run = results[primary]
    kernels, kb, s = main_run["kernels"], main_run["kb"], main_run["sizes"]
    # the longest kernel among those with a byte model (the small ones carry ~no bytes)
    dom = max((k for k in kernels if k in kb), key=lambda k: kernels[k]["mean_us"])
    dom_us = kernels[dom]["mean_us"]
    achieved = kb[dom] / (dom_us * 1e-6) / 1e9
    traffic = traffic_for(dom)
    ms = main_run["ms"]
    out = {
        "metric": METRIC,
        "value": round(main_run["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(main_run["ms_med"], 4),
        "ms_per_step_min": round(main_run["ms_min"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (planted low-rank + 0.05*N(0,1) worker noise, drawn on device)",
        "config": {"workload": "resnet18_cifar_shapes", "rank": wl.rank, "workers": W,
                   "matrices": s["n_matrices"], "uncompressed_tensors": s["n_vectors"],
                   "params": s["numel"], "grad_bytes_per_step": main_run["grad_bytes"],
                   "plan_flags": {"plain": "0", "carry": "PSGD_FLAG_CARRY_ERROR_MEAN",
                                  "deferred": "PSGD_FLAG_DEFERRED_ERROR",
                                  "local": "PSGD_FLAG_LOCAL_Q_ERROR"}[primary]},
        "pct_hbm_peak": round(main_run["pct"], 2),
        "model_bytes_per_step": s["model_bytes"],
        "kernel_bytes_per_step": main_run["own_bytes"],
        "pct_hbm_peak_kernel_bytes": round(main_run["pct_own"], 2),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": kb[dom], "mean_us": dom_us},
        "kernels": kernels,
        "ms_per_step_with_kernel_events": round(main_run["ms_timed"], 4),
        "ms_per_step_graph_replay": round(main_run["ms_graph"], 4) if main_run["ms_graph"] else None,
        "stream_copy_GBps": round(copy_gbs, 1),
    }
    out["variants"] = {n: {"value": round(r["value"], 2), "ms_per_step": round(r["ms"], 4),
                           "pct_hbm_peak": round(r["pct"], 2),
                           "kernel_bytes_per_step": r["own_bytes"],
                           "pct_hbm_peak_kernel_bytes": round(r["pct_own"], 2),
                           "kernels_mean_us": {k: v["mean_us"] for k, v in r["kernels"].items()}}
                       for n, r in results.items() if n != primary}
    if args.mode == "all":
        out["rtopk"] = measure_rtopk()
        out["atomo"] = measure_atomo()
        if not args.no_configs:
            out["other_configs"] = config_timings(torch, psgd, WL, dev, args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
