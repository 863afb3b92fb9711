#!/usr/bin/env python3
"""Throughput of exact Lloyd k-means on one MI355X.

A step is one Lloyd iteration over the whole workload: centroid prep, the
fused assignment (with the objective), the counting argsort of the labels,
the segmented reduction and the divide -- all in the HIP kernels behind the
C ABI.  Inputs are resident in device memory before the timed region.

Prints one JSON line: iterations/s, the assignment kernel against its
roofline (HIP events around every assignment in the timed region), the
update's bandwidth, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Lloyd iter/s at N=1M K=8192 d=128 fp16; assign TFLOP/s, update GB/s"
PEAK_MFMA_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}  # dense MI355X matrix-core peaks
PEAK_HBM_GBS = 8000.0
# One float32 vector operation per lane per clock, unpacked: 256 CUs x 4 SIMDs
# x 16 lanes x 2.4 GHz (the library is built without packed fp32).
PEAK_VALU_GOPS = 256 * 4 * 16 * 2.4
# Algorithmic float32 operations per point per scalar Lloyd iteration: the two
# bracketing distances (2 sub, 2 mul) and their comparison, the weighted sum
# and weight sum (fma, add), and the objective term (fma).
OPS_1D_PER_POINT = 8
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
# the sources of the assignment kernel: a traffic figure holds while they are unchanged
ASSIGN_SRC = [os.path.join(ROOT, "exact_lloyd_means_03_amd", "csrc", f) for f in ("assign_mfma.hip", "common.h")]


def update_bytes(wl) -> float:
    """Algorithmic bytes of one update: points gathered once, labels read once,
    perm written and read once, weights (if any), old + new centroids, counts."""
    B, N, d, K, s = wl.B, wl.N, wl.d, wl.K, ELEM_BYTES[wl.dtype]
    w = 4 * B * N if wl.weighted else 0
    return B * N * d * s + 4 * B * N + 8 * B * N + w + 8 * B * K * d + 4 * B * K


def assign_bytes(wl) -> float:
    """Algorithmic bytes of one assignment: points once, labels written, centroids once."""
    B, N, d, K, s = wl.B, wl.N, wl.d, wl.K, ELEM_BYTES[wl.dtype]
    w = 4 * B * N if wl.weighted else 0
    return B * N * (d * s + 4) + w + B * K * d * 4


def _src_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _traffic(wl):
    """HBM bytes per assignment launch from the committed rocprofv3 counter
    summary of this workload, if it was taken with the current kernel source."""
    try:
        t = json.load(open(os.path.join(TRAFFIC_DIR, f"assign_traffic__{wl.name}.json")))
    except (OSError, ValueError):
        return None
    if t.get("workload") != wl.name or t.get("kernel_src_sha") != _src_hash(ASSIGN_SRC):
        return None
    return t.get("bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (the "model name" line that lscpu also shows)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(p, target_s: float):
    """Time the CPU oracle on a bounded sample and extrapolate to one Lloyd
    iteration over the whole workload: with one batch, n points against all
    K centroids (assignment) plus their update, scaled linearly in N; with
    several batches, whole batches (all their points), scaled linearly in B."""
    import numpy as np

    import oracle
    import workloads

    wl = p.wl
    bits = workloads.raw_bits(p.x)
    C = p.init.numpy()
    rng = np.random.default_rng(12345)

    def run_points(n):
        idx = np.sort(rng.choice(wl.N, size=n, replace=False))
        X = oracle.decode(bits[0:1, idx], wl.dtype)
        Chat = oracle.decode(oracle.round_to(C[0:1], wl.dtype), wl.dtype)
        w = None if p.w is None else p.w[0:1, idx].numpy()
        t0 = time.perf_counter()
        lab, d1, d2 = oracle.assign(X, Chat)
        oracle.update(X, w, lab, C[0:1])
        return time.perf_counter() - t0

    def run_batches(nb):
        rows = np.sort(rng.choice(wl.B, size=nb, replace=False))
        X = oracle.decode(bits[rows], wl.dtype)
        Chat = oracle.decode(oracle.round_to(C[rows], wl.dtype), wl.dtype)
        w = None if p.w is None else p.w[rows].numpy()
        t0 = time.perf_counter()
        lab, d1, d2 = oracle.assign(X, Chat)
        oracle.update(X, w, lab, C[rows])
        return time.perf_counter() - t0

    if wl.B == 1:
        total, run = wl.N, run_points
    else:
        total, run = wl.B, run_batches
    n = min(total, 1 if wl.B > 1 else 256)
    t = run(n)
    while t < 0.5 and n < total:
        n = min(total, n * 4)
        t = run(n)
    if n < total:
        n = int(min(total, max(n, n * target_s / max(t, 1e-9))))
        t = run(n)
    per_iter = t * (total / n)
    what = (f"{n} of {wl.N} points" if wl.B == 1 else f"{n} of {wl.B} batches ({wl.N} points each)")
    return {
        "value": 1.0 / per_iter,
        "unit": "iter/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{what}: one oracle assignment against all K={wl.K} centroids plus the update, "
                   f"{t:.2f} s, extrapolated linearly to one iteration over all {wl.B * wl.N} points"),
    }


def bench_update(km, wl, reps: int = 5) -> dict:
    """The update stage (kmeans_update: argsort, segmented reduction, divide)
    on a workload's points with the labels of its first assignment: device
    time per call from HIP events around each of `reps` calls, against the
    update's algorithmic bytes and the HBM peak."""
    import torch

    import workloads

    p = workloads.generate(wl)
    dev = torch.device("cuda", 0)
    x = p.x.to(dev)
    C = p.init.to(dev)
    B, N, d, K = wl.B, wl.N, wl.d, wl.K
    ws = km.workspace(B, N, d, K, x.dtype, dev)
    labels, _, _ = km.kmeans_assign(x, C, ws=ws)
    c_new = torch.empty_like(C)
    counts = torch.empty((B, K), dtype=torch.int32, device=dev)
    km.kmeans_update(x, labels, C, c_new=c_new, counts=counts, ws=ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for r in range(reps):
        km.kmeans_update(x, labels, C, c_new=c_new, counts=counts, ws=ws)
        ev[r + 1].record()
    torch.cuda.synchronize()
    ms = sum(ev[r].elapsed_time(ev[r + 1]) for r in range(reps)) / reps
    ub = update_bytes(wl)
    out = {"workload": wl.name, "avg_ms": ms, "calls": reps, "algorithmic_bytes": ub,
           "GB/s": ub / (ms * 1e-3) / 1e9, "frac_hbm": ub / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "largest_cluster": int(counts.max()),
           "timing": "HIP events around each kmeans_update call (argsort, segmented reduction, divide)"}
    del x, C, ws, labels, c_new, counts
    torch.cuda.empty_cache()
    return out


def bench_graph_fit(km, x, init, w, steps: int, ws, reps: int = 20) -> dict:
    """Launch overhead of a small fit: the same kmeans_fit of `steps`
    iterations called eagerly and replayed from a HIP graph it was captured
    into (the library enqueues kernels only, so the whole fit captures),
    `reps` times each between synchronizations, wall clock."""
    import torch

    B, K, d = init.shape
    N = x.shape[1]
    cen = torch.empty_like(init)
    lab = torch.empty((B, N), dtype=torch.int32, device=x.device)
    cnt = torch.empty((B, K), dtype=torch.int32, device=x.device)
    obj = torch.empty((B, steps), dtype=torch.float64, device=x.device)

    def fit():
        km.kmeans_fit(x, init, steps, weights=w, centroids=cen, labels=lab, counts=cnt, objective=obj, ws=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fit()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fit()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fit()
    torch.cuda.synchronize()
    eager = time.perf_counter() - t0
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    graph = time.perf_counter() - t0
    return {"iterations_per_fit": steps, "fits": reps, "eager_ms_per_iter": eager / (reps * steps) * 1e3,
            "graph_ms_per_iter": graph / (reps * steps) * 1e3, "graph_iter_per_s": reps * steps / graph,
            "timing": "wall clock over `fits` back-to-back fits, eager calls vs replays of one captured fit"}


def bench_fit_1d(args, km, wl, p, x, w, C):
    """Scalar rows: kmeans_fit runs every iteration of rows of up to 8192
    points with K <= 16 in one launch, so a step is one iteration inside
    that launch.  The warmup is a
    fit of W iterations; the timed region is one fit of exactly K iterations
    from the same initial centroids (the wall clock between synchronizations);
    the roofline's launch time is a second such fit timed with HIP events on
    the launch stream behind a spin kernel."""
    import torch

    B, N, d, K = wl.B, wl.N, wl.d, wl.K
    init = C.clone()
    if args.warmup > 0:
        km.kmeans_fit(x, init, args.warmup, weights=w)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, _, _, J_lloyd = km.kmeans_fit(x, init, args.steps, weights=w)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # device time of the same fit: a spin kernel holds the stream while the
    # call is prepared on the host, so the events see only the launch
    fit_ms = _device_ms(lambda: km.kmeans_fit(x, init, args.steps, weights=w), 1)
    ops = OPS_1D_PER_POINT * B * N * args.steps
    achieved = ops / (fit_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": args.steps / elapsed,
        "unit": "iter/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "N": N, "d": d, "K": K, "point_dtype": wl.dtype,
                   "weighted": wl.weighted, "init": wl.init, "path": "whole fit in one launch"},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_VALU_GOPS, "unit": "Gop/s",
                     "frac": achieved / PEAK_VALU_GOPS, "traffic": None,
                     "kernel": ("k_fit_1d_wave" if N <= 4096 else "k_fit_1d_rows") if N <= 8192 and K <= 16
                     else "kmeans_fit",
                     "algorithmic_per_launch": ops, "avg_launch_ms": fit_ms},
        "cpu_baseline": None,
    }
    out["steps_1d"] = bench_steps_1d(km, wl, x, w, C)
    if N <= 4096:
        out["optimal_1d"] = bench_optimal_1d(km, wl, x, w, J_lloyd[:, -1])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def _device_ms(fn, reps: int) -> float:
    """Device time per call of fn, with the calls queued back to back: a spin
    kernel holds the stream while they are enqueued, so host-side launch
    overhead does not open gaps between them."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(5e6))
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_steps_1d(km, wl, x, w, C, reps: int = 10) -> dict:
    """The single assignment (with the weighted objective) and update calls on
    the same rows, each against HBM: the bytes they must move are the points,
    the weights and the labels once each, plus the centroids (the update needs
    no argsort for K <= 16, so no permutation bytes are counted)."""
    import torch

    B, N, K, s = wl.B, wl.N, wl.K, ELEM_BYTES[wl.dtype]
    labels = torch.empty((B, N), dtype=torch.int32, device=x.device)
    counts = torch.empty((B, K), dtype=torch.int32, device=x.device)
    obj = torch.empty((B,), dtype=torch.float64, device=x.device)
    c_new = torch.empty_like(C)
    ws = km.workspace(B, N, 1, K, x.dtype, x.device)
    wb = 4 * B * N if w is not None else 0

    def assign():
        km.kmeans_assign(x, C, weights=w, labels=labels, objective=obj, ws=ws)

    def update():
        km.kmeans_update(x, labels, C, weights=w, c_new=c_new, counts=counts, ws=ws)

    assign()
    update()
    a_ms, u_ms = _device_ms(assign, reps), _device_ms(update, reps)
    a_bytes = B * N * (s + 4) + wb + 4 * B * K
    u_bytes = B * N * (s + 4) + wb + 8 * B * K + 4 * B * K
    out = {}
    for name, ms, nb in (("assign", a_ms, a_bytes), ("update", u_ms, u_bytes)):
        gbs = nb / (ms * 1e-3) / 1e9
        out[name] = {"avg_ms": ms, "algorithmic_bytes": nb, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}
    return out


def bench_optimal_1d(km, wl, x, w, J_lloyd, reps: int = 3) -> dict:
    """The globally optimal 1D clustering of the same rows (kmeans_optimal_1d,
    one launch): device time per call, and its objective next to the Lloyd
    fit's last objective from the same rows."""
    import torch

    B, N, K = wl.B, wl.N, wl.K
    L = km.load()
    ws = torch.empty(max(int(L.kmeans_optimal_1d_workspace_bytes(B, N, K)), 256), dtype=torch.uint8,
                     device=x.device)
    cen = torch.empty((B, K), dtype=torch.float32, device=x.device)
    lab = torch.empty((B, N), dtype=torch.int32, device=x.device)
    cnt = torch.empty((B, K), dtype=torch.int32, device=x.device)
    J = torch.empty((B,), dtype=torch.float64, device=x.device)

    def run():
        km.kmeans_optimal_1d(x, K, weights=w, centroids=cen, labels=lab, counts=cnt, objective=J, ws=ws)

    run()
    ms = _device_ms(run, reps)
    Jm, Jl = float(J.mean()), float(J_lloyd.mean())
    return {"kernel": "k_optimal_1d", "avg_ms": ms, "rows_per_s": B / (ms * 1e-3), "J_mean": Jm,
            "lloyd_J_mean": Jl, "J_over_lloyd": Jm / Jl}


def bench_stream(args, km, wl):
    """A workload whose points stay in pinned host memory (kmeans_fit_stream):
    a step is one Lloyd iteration including the host-to-device copy of every
    point.  The line also gives the bare copy rate, the same fit with the
    points in device memory, and how much of the shorter of the two the
    streamed iteration hides."""
    import torch

    import workloads

    N, d, K = wl.N, wl.d, wl.K
    chunk = args.chunk
    x_host, init = workloads.generate_host(wl)
    nbytes = x_host.numel() * x_host.element_size()
    # the streamed fit first (a long run before it would leave the chip
    # hotter): W warmup iterations, then exactly K timed ones
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    L = km.load()
    xt = {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype]
    ws = torch.empty(max(int(L.kmeans_stream_workspace_bytes(N, d, K, xt, chunk)), 256), dtype=torch.uint8,
                     device="cuda")
    if args.warmup > 0:
        km.kmeans_fit_stream(x_host, init, args.warmup, chunk=chunk, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    _, _, _, J = km.kmeans_fit_stream(x_host, init, args.steps, chunk=chunk, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    it_ms = e0.elapsed_time(e1) / args.steps
    # then the bare copy, and the fit with the points already in device memory
    x_dev = torch.empty((1, N, d), dtype=x_host.dtype, device="cuda")
    x_dev[0].copy_(x_host, non_blocking=True)
    torch.cuda.synchronize()
    e0.record()
    x_dev[0].copy_(x_host, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1)
    ws_dev = km.workspace(1, N, d, K, x_dev.dtype, x_dev.device)
    km.kmeans_fit(x_dev, init[None], 1, ws=ws_dev)
    torch.cuda.synchronize()
    e0.record()
    km.kmeans_fit(x_dev, init[None], args.steps, ws=ws_dev)
    e1.record()
    torch.cuda.synchronize()
    dev_ms = e0.elapsed_time(e1) / args.steps
    del x_dev, ws_dev
    torch.cuda.empty_cache()
    flops = 2.0 * N * K * d
    achieved = flops / (it_ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    out = {
        "metric": "out-of-core Lloyd iter/s (points in pinned host memory, host-to-device copies included)",
        "value": args.steps / elapsed,
        "unit": "iter/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": 1, "N": N, "d": d, "K": K, "point_dtype": wl.dtype, "init": wl.init,
                   "chunk": chunk, "host_bytes": nbytes},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": None, "kernel": "k_assign_mfma (streamed)", "algorithmic_per_launch": flops,
                     "avg_launch_ms": it_ms},
        "transfer": {"bytes_per_iter": nbytes, "bare_copy_ms": copy_ms, "GB/s": nbytes / (copy_ms * 1e-3) / 1e9},
        "device_memory_fit_ms_per_iter": dev_ms,
        # 1: the streamed iteration takes max(copy, kernels); 0: their sum
        "hidden": (copy_ms + dev_ms - it_ms) / min(copy_ms, dev_ms),
        "objective_last": float(J[-1]),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import types
        p = types.SimpleNamespace(wl=wl, x=x_host[None], w=None, init=init[None].cpu())
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_emeans(p, target_s: float):
    """Time the oracle's e-means on a bounded sample: n points as one batch
    (one step against all K centroids, with the moving average and the
    splits), scaled linearly to one epoch over all N points."""
    import numpy as np

    import oracle
    import workloads

    wl = p.wl
    bits = workloads.raw_bits(p.x)[0]
    init = p.init[0].numpy()
    u = workloads.emeans_uniforms(wl.seed, 1, wl.K)

    def run(n):
        t0 = time.perf_counter()
        oracle.emeans(bits[:n], wl.dtype, init, n, 1, wl.em_alpha0, wl.em_floor, wl.em_dead_frac, wl.em_eps, u)
        return time.perf_counter() - t0

    n = 256
    t = run(n)
    while t < 0.5 and n < wl.N:
        n = min(wl.N, n * 4)
        t = run(n)
    if n < wl.N:
        n = int(min(wl.N, max(n, n * target_s / max(t, 1e-9))))
        t = run(n)
    per_epoch = t * wl.N / n
    return {
        "value": 1.0 / per_epoch,
        "unit": "epochs/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"the first {n} of {wl.N} points as one e-means step against all K={wl.K} centroids "
                   f"(assignment, moving average, splits), {t:.2f} s, extrapolated linearly to one epoch"),
    }


def bench_emeans(args, km, wl):
    """e-means (kmeans_emeans): a step is one whole e-means run of
    wl.em_epochs epochs in batches of wl.em_batch points, points resident in
    device memory.  `value` is epochs/s.  Outside the timed region the line
    also gives the mean squared error of the final centroids after 1..E
    epochs next to Lloyd's after wl.n_iter iterations from the same init,
    both fits' times, and the assignment kernel on one batch against its
    matrix-core roofline."""
    import torch

    import workloads

    dev = torch.device("cuda", 0)
    p = workloads.generate(wl)
    x = p.x[0].to(dev)
    init = p.init[0].to(dev)
    N, d, K, batch, E = wl.N, wl.d, wl.K, wl.em_batch, wl.em_epochs
    T = km.emeans_steps(N, batch, E)
    u = torch.from_numpy(workloads.emeans_uniforms(wl.seed, T, K)).to(dev)
    L = km.load()
    xt = {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype]
    ws = torch.empty(max(int(L.kmeans_emeans_workspace_bytes(N, d, K, xt, batch)), 256), dtype=torch.uint8,
                     device=dev)
    cen = torch.empty_like(init)
    counts = torch.empty((K,), dtype=torch.int32, device=dev)

    def run(epochs):
        t_ = km.emeans_steps(N, batch, epochs)
        obj = torch.empty((t_,), dtype=torch.float64, device=dev)
        km.kmeans_emeans(x, init, batch, epochs, wl.em_alpha0, wl.em_floor, wl.em_dead_frac, wl.em_eps,
                         uniforms=u[:t_], centroids=cen, counts=counts, objective=obj, ws=ws)
        return obj

    for _ in range(args.warmup):
        run(E)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        run(E)
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    run_ms = e0.elapsed_time(e1) / args.steps

    # quality: the mean squared error of the final centroids over all points
    ws_a = km.workspace(1, N, d, K, x.dtype, dev)
    xb = x[None]
    o = torch.empty((1,), dtype=torch.float64, device=dev)

    def mse(c):
        km.kmeans_assign(xb, c[None], objective=o, ws=ws_a)
        return float(o[0]) / N

    em_mse, em_ms = [], []
    for e in range(1, E + 1):
        run(e)
        torch.cuda.synchronize()
        e0.record()
        run(e)
        e1.record()
        torch.cuda.synchronize()
        em_ms.append(e0.elapsed_time(e1))
        em_mse.append(mse(cen))
    ws_l = km.workspace(1, N, d, K, x.dtype, dev)
    km.kmeans_fit(xb, init[None], 1, ws=ws_l)
    torch.cuda.synchronize()
    e0.record()
    cl, _, _, Jl = km.kmeans_fit(xb, init[None], wl.n_iter, ws=ws_l)
    e1.record()
    torch.cuda.synchronize()
    lloyd_ms = e0.elapsed_time(e1)
    lloyd_mse = mse(cl[0])
    match = next((e + 1 for e, m in enumerate(em_mse) if m <= lloyd_mse), None)

    # the dominant kernel: the assignment of one full batch, timed on its own
    xs = x[None, :batch]
    lab = torch.empty((1, batch), dtype=torch.int32, device=dev)
    ws_b = km.workspace(1, batch, d, K, x.dtype, dev)
    reps = 20
    km.kmeans_assign(xs, cen[None], labels=lab, ws=ws_b)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        km.kmeans_assign(xs, cen[None], labels=lab, ws=ws_b)
    e1.record()
    torch.cuda.synchronize()
    assign_ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * batch * K * d
    achieved = flops / (assign_ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    out = {
        "metric": "e-means epochs/s (mini-batch moving-average k-means, all points resident in HBM)",
        "value": args.steps * E / elapsed,
        "unit": "epochs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "N": N, "d": d, "K": K, "point_dtype": wl.dtype, "init": wl.init,
                   "batch": batch, "epochs": E, "steps_per_run": T, "alpha0": wl.em_alpha0,
                   "floor": wl.em_floor, "dead_frac": wl.em_dead_frac, "eps": wl.em_eps},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": _traffic(wl),
                     "kernel": "k_assign_mfma + k_assign_merge (one batch, centroid tiles in slices)",
                     "algorithmic_per_launch": flops,
                     "avg_launch_ms": assign_ms},
        "run_ms_event": run_ms,
        "quality": {"emeans_mse_by_epochs": em_mse, "emeans_ms_by_epochs": em_ms,
                    "lloyd_iters": wl.n_iter, "lloyd_mse": lloyd_mse, "lloyd_ms": lloyd_ms,
                    "lloyd_objective_last_iter": float(Jl[0, -1]) / N,
                    "epochs_to_match_lloyd": match,
                    "speedup_at_match": (lloyd_ms / em_ms[match - 1]) if match else None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_emeans(p, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--chunk", type=int, default=1 << 22, help="points per host-to-device copy (host workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-zipf-update", action="store_true",
                    help="skip the 33M-point update measurement that the headline line carries")
    ap.add_argument("--points", type=int, default=0,
                    help="run the workload with this many points per problem instead (profiling runs whose "
                         "counters must stay below 2^31 per dispatch); the line then names the reduced size")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the batched problems are independent per GPU)", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_lloyd_means_03_amd as km
    import workloads

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 5}))
        return
    km.load()  # raises if the HIP library is missing
    name = args.workload or workloads.HEADLINE
    wl = workloads.WORKLOADS[name]
    if args.points:
        wl = wl.replace(name=f"{wl.name}@N={args.points}", N=args.points)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if wl.host:
        return bench_stream(args, km, wl)
    if wl.em_batch:
        return bench_emeans(args, km, wl)
    if wl.device_gen:
        p = None  # made on the GPU; no host copy for the CPU baseline
        x, C = workloads.generate_device(wl)
        w = None
    else:
        p = workloads.generate(wl)
        x = p.x.to(dev)
        w = None if p.w is None else p.w.to(dev)
        C = p.init.to(dev).clone()
    B, N, d, K = wl.B, wl.N, wl.d, wl.K
    ws = km.workspace(B, N, d, K, x.dtype, dev)
    labels = torch.empty((B, N), dtype=torch.int32, device=dev)
    counts = torch.empty((B, K), dtype=torch.int32, device=dev)
    obj = torch.empty((B, max(args.warmup, 1)), dtype=torch.float64, device=dev)

    if d == 1:
        return bench_fit_1d(args, km, wl, p, x, w, C)

    # warmup: W iterations of the fit, continued by the timed fit from where
    # they left the centroids
    if args.warmup > 0:
        km.kmeans_fit(x, C, args.warmup, weights=w, centroids=C, labels=labels, counts=counts,
                      objective=obj[:, :args.warmup].contiguous(), ws=ws)
    torch.cuda.synchronize()

    # The timed region is ONE kmeans_fit call of exactly K iterations: each
    # iteration is prep (fused into the previous divide), the assignment with
    # the objective, the argsort, the segmented reduction and the divide.
    K_steps = args.steps
    objK = torch.empty((B, K_steps), dtype=torch.float64, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    km.kmeans_fit(x, C, K_steps, weights=w, centroids=C, labels=labels, counts=counts, objective=objK, ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    # The split of an iteration into assignment and update comes from a second
    # fit of K iterations (continuing from the first one's centroids) in which
    # the library records a pair of events around every iteration's
    # assignment kernel on the launch stream.  Each timing event costs a few
    # microseconds of its own, which is why the throughput above is taken
    # from the fit without them.
    events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K_steps)]
    for e in events:
        e.record()  # creates the events; the fit re-records them in place
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    km.kmeans_fit(x, C, K_steps, weights=w, centroids=C, labels=labels, counts=counts, objective=objK, ws=ws,
                  assign_events=events)
    e_end.record()
    torch.cuda.synchronize()
    elapsed_events = time.perf_counter() - t2
    assign_each = [events[2 * k].elapsed_time(events[2 * k + 1]) for k in range(K_steps)]
    # the rest of an iteration: from the end of its assignment to the start of
    # the next one (objective reduction, argsort, segmented reduction, divide
    # fused with the next prep); the last iteration ends with the call
    rest_each = [events[2 * k + 1].elapsed_time(events[2 * k + 2]) for k in range(K_steps - 1)]
    rest_each.append(events[2 * K_steps - 1].elapsed_time(e_end))
    assign_ms = sum(assign_each) / K_steps
    update_ms = sum(rest_each) / K_steps
    bound, unit = "mfma", "TFLOP/s"
    algo = 2.0 * B * N * K * d
    achieved = algo / (assign_ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    ub = update_bytes(wl)
    out = {
        "metric": METRIC,
        "value": K_steps / elapsed,
        "unit": "iter/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / K_steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "N": N, "d": d, "K": K, "point_dtype": wl.dtype,
                   "weighted": wl.weighted, "init": wl.init, "step": "one kmeans_fit call of `steps` iterations"},
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": _traffic(wl),
                     "kernel": "k_assign_mfma",
                     "algorithmic_per_launch": algo, "avg_launch_ms": assign_ms,
                     "timing": "HIP events recorded by the library around each assignment kernel in a second fit "
                               "of the same steps"},
        "ms_per_step_with_events": elapsed_events / K_steps * 1e3,
        "update": {"avg_ms": update_ms, "algorithmic_bytes": ub, "GB/s": ub / (update_ms * 1e-3) / 1e9,
                   "frac_hbm": ub / (update_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                   "timing": "events: end of one assignment to the start of the next (objective reduction, "
                             "argsort, segmented reduction, divide + next prep)"},
        "cpu_baseline": None,
    }
    if B * N * K * d <= (1 << 30):  # launch-bound sizes: the same fit replayed from a HIP graph
        out["graph"] = bench_graph_fit(km, x, C, w, K_steps, ws)
    del x, w, ws, labels, counts
    torch.cuda.empty_cache()
    if not args.no_zipf_update and wl.name == workloads.HEADLINE and not args.points:
        out["update_zipf"] = bench_update(km, workloads.WORKLOADS["zipf-n32m-k4096-d128-bf16"])
    if not args.no_cpu_baseline and p is not None:
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
