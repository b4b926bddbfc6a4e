#!/usr/bin/env python3
"""Benchmark of the Dion step on one MI355X.

A "step" is one Dion update of every matrix of the workload (all stacks),
with gradients already resident in HBM.  The default workload is the
rank-fraction-1/4 attention stack: 24 fp32 matrices of 1024 x 1024 at r = 256
with low-rank-plus-noise gradients (see workloads/).  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload 1..5] [--no-cpu-baseline]

The K timed steps run twice: eagerly (one host launch per kernel, with the library's phase
events) and as replays of the same steps captured in HIP graphs (one graph per resident
gradient).  The replays set the value; both times are reported ("eager_ms_per_step",
"graph_ms_per_step"), and --eager times the eager steps only.

Metric: updates/s (steps per second over the whole workload), with the
effective parameter bandwidth (algorithmic bytes / step time) and its share of
the 8 TB/s HBM peak alongside.  The "roofline" entry times the dominant kernel
live (HIP events recorded by the library at its phase boundaries, on the
stream the kernels run on); the "cpu_baseline" entry times the fp64 oracle on
the host cores over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"f64": 78.6, "f32": 157.3, "bf16": 2500.0}


def algorithmic_bytes(wl) -> float:
    """Per step: read G, read+write M (fp32), read+write X, read+write Q (fp32)."""
    bx = 2 if wl.x_dtype == "bf16" else 4
    tot = 0.0
    for g in wl.groups:
        tot += g.batch * (g.m * g.n * (bx + 8 + 2 * bx) + 8 * g.n * g.rank)
    return tot


def algorithmic_flops(wl) -> float:
    """Per step: four rank-r contractions plus CholeskyQR2 (two Grams, Cholesky, solves)."""
    tot = 0.0
    for g in wl.groups:
        m, n, r = g.m, g.n, g.rank
        tot += g.batch * (8.0 * m * n * r + 6.0 * m * r * r + 2.0 * r ** 3 / 3.0)
    return tot


def kernel_source_hash(root: str) -> str:
    """sha256 over the kernel and ABI sources the shared library is built from."""
    import glob
    import hashlib
    files = sorted(f for f in glob.glob(os.path.join(root, "rank_orthonormalized_optimizer_amd", "csrc", "*"))
                   if f.endswith((".hip", ".hpp", ".h", ".cpp")))
    files.append(os.path.join(root, "include", "dion.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, phase: str):
    """HBM bytes per launch of the phase's kernel, from the rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary in profiles/traffic.json (already scaled by the copy-kernel calibration), or None
    when there is none for this kernel or it was taken on other kernel sources."""
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, "profiles", "traffic.json")) as fh:
            ent = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not ent or ent.get("source_sha256") != kernel_source_hash(root):
        return None
    ph = ent.get("phases", {}).get(phase)
    return None if ph is None else ph["bytes_per_launch"]


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        return int(max(n)) if n else (os.cpu_count() or 1)
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(wl, budget_s: float) -> dict:
    """The fp64 oracle as it stands, on the host cores, over a bounded sample of the workload.

    Every matrix of every stack is stepped once (step-1 inputs); the per-stack pass is
    repeated while the budget lasts, then the mean time per full step is reported.
    Stacks whose single matrix already exceeds the budget are sampled: the per-matrix
    time of the matrices that fit is scaled to the whole stack.
    """
    import numpy as np

    import workloads as W
    from oracle import dion_step
    t_all = time.perf_counter()
    per_group = []
    for gi, g in enumerate(wl.groups):
        X, M, Q = W.make_state(wl, gi)
        G = W.make_grad(wl, gi, 1)
        args = [(W.to_f64(X[i], wl.x_dtype), W.to_f64(G[i], wl.g_dtype), M[i].astype(np.float64),
                 Q[i].astype(np.float64)) for i in range(g.batch)]
        share = budget_s / len(wl.groups)
        times, t0 = [], time.perf_counter()
        while True:
            for i in range(g.batch):
                t1 = time.perf_counter()
                dion_step(*args[i], wl.mu, wl.lr, wl.eps)
                times.append(time.perf_counter() - t1)
                if time.perf_counter() - t0 > share and len(times) >= 1:
                    break
            if time.perf_counter() - t0 > share:
                break
        per_group.append((g, float(np.mean(times)), len(times)))
    step_s = sum(g.batch * t for g, t, _ in per_group)
    sample = "; ".join(f"{k} matrix steps of the {g.batch}x{g.m}x{g.n} r={g.rank} stack"
                       for g, _, k in per_group)
    return {"value": 1.0 / step_s, "unit": "updates/s", "cores": blas_threads(), "kind": "oracle",
            "sample": sample + f" (step-1 inputs, fp64 numpy/OpenBLAS; mean time per matrix x stack size; "
                               f"{time.perf_counter() - t_all:.1f} s of CPU work)",
            "s_per_step": step_s}


EW_N = 64 << 20    # elements of the element-wise measurement (256 MiB per fp32 array)
EW_BYTES = {"adamw": 28, "lion": 20}   # algorithmic bytes per fp32 element: reads p, g, m(, v); writes p, m(, v)


def elementwise_block(dev, stream, iters: int = 20, cpu_s: float = 3.0, with_cpu: bool = True) -> dict:
    """AdamW and Lion (the element-wise optimizers for the parameters Dion does not take) on one
    fp32 array of EW_N elements resident in HBM: achieved GB/s against the 8 TB/s HBM peak,
    timed with events on the launch stream, and the fp64 oracle on a bounded host sample."""
    import numpy as np
    import torch

    import rank_orthonormalized_optimizer_amd as dion
    gen = torch.Generator(device=dev).manual_seed(7)
    p = (0.02 * torch.randn(EW_N, generator=gen, device=dev)).contiguous()
    g = (1e-2 * torch.randn(EW_N, generator=gen, device=dev)).contiguous()
    m = torch.zeros(EW_N, device=dev)
    v = torch.zeros(EW_N, device=dev)
    out = {"n": EW_N, "dtype": "f32", "data": "synthetic"}
    runs = {"adamw": lambda t: dion.adamw_step_(p, g, m, v, t, 1e-3, 0.9, 0.999, 1e-8, 0.1, stream=stream),
            "lion": lambda t: dion.lion_step_(p, g, m, 3e-4, 0.9, 0.99, 0.1, stream=stream)}
    for name, run in runs.items():
        for t in range(1, 4):
            run(t)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for t in range(4, 4 + iters):
            run(t)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        gbs = EW_BYTES[name] * EW_N / (ms * 1e-3) / 1e9
        out[name] = {"ms_per_step": ms, "effective_GBps": gbs, "bytes_per_element": EW_BYTES[name],
                     "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": gbs / HBM_PEAK_GBS}}
    del p, g, m, v
    if with_cpu:
        from oracle.elementwise_oracle import adamw_step, lion_step
        k = 1 << 22
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([7, k])))
        hp, hg = 0.02 * rng.standard_normal(k), 1e-2 * rng.standard_normal(k)
        hm, hv = np.zeros(k), np.zeros(k)
        for name in ("adamw", "lion"):
            reps, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < cpu_s / 2:
                if name == "adamw":
                    adamw_step(hp, hg, hm, hv, 1, 1e-3, 0.9, 0.999, 1e-8, 0.1)
                else:
                    lion_step(hp, hg, hm, 3e-4, 0.9, 0.99, 0.1)
                reps += 1
            per_elem = (time.perf_counter() - t0) / (reps * k)
            out[name]["cpu_baseline"] = {"value": EW_BYTES[name] / per_elem / 1e9, "unit": "GB/s", "cores": 1,
                                         "kind": "oracle",
                                         "sample": f"{reps} steps of {k} elements (fp64 numpy, one thread)"}
    return out


SPECTRAL_CASES = ((24, 256), (8, 4096))   # (matrices, r): the Gram shapes of the attention and full-rank stacks
SPECTRAL_K, SPECTRAL_ITERS = 32, 10


def spectral_block(dev, stream, reps: int = 10, with_cpu: bool = True) -> dict:
    """The multi-power-iteration lambda_max estimate (dion_lambda_max_batched) on fp64 Gram
    stacks A^T A resident in HBM, 32 start vectors, 10 normalized products.  The product kernel
    is priced against the fp64 vector peak: 2 r^2 k flops per matrix and product, its time the
    difference between calls with 10 and with 0 iterations (10 more product launches), measured
    with events on the launch stream.  The fp64 oracle runs on one matrix of each stack."""
    import numpy as np
    import torch

    import rank_orthonormalized_optimizer_amd as dion
    out = {"k": SPECTRAL_K, "iters": SPECTRAL_ITERS, "dtype": "f64", "data": "synthetic", "cases": []}
    for b, r in SPECTRAL_CASES:
        gen = torch.Generator(device=dev).manual_seed(41 + r)
        A = torch.randn(b, r + 8, r, generator=gen, device=dev, dtype=torch.float64)
        Wm = torch.matmul(A.transpose(1, 2).contiguous(), A).contiguous()   # input preparation only
        del A
        lam = torch.empty(b, dtype=torch.float64, device=dev)

        def timed(iters):
            for _ in range(2):
                dion.lambda_max_(Wm, k=SPECTRAL_K, iters=iters, out=lam, stream=stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                dion.lambda_max_(Wm, k=SPECTRAL_K, iters=iters, out=lam, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        ms_full, ms_zero = timed(SPECTRAL_ITERS), timed(0)
        prod_ms = max(ms_full - ms_zero, 0.0) / SPECTRAL_ITERS
        flops = 2.0 * r * r * SPECTRAL_K * b
        tf = flops / (prod_ms * 1e-3) / 1e12 if prod_ms > 0 else 0.0
        case = {"workload": f"{b}x{r}x{r} Gram stack", "ms_per_call": ms_full,
                "calls_per_s": 1e3 / ms_full, "product_launch_ms": prod_ms,
                "roofline": {"bound": "alu", "kernel": "mpi_product_kernel", "achieved": tf,
                             "peak": PEAK_TFLOPS["f64"], "unit": "TFLOP/s", "frac": tf / PEAK_TFLOPS["f64"],
                             "flops_per_launch": flops,
                             "traffic": measured_traffic(f"spectral-{b}x{r}x{r}", "mpi_product_kernel"),
                             "traffic_unit": "bytes/launch",
                             "algorithmic_bytes_per_launch": b * (8.0 * r * r + 16.0 * r * SPECTRAL_K)}}
        if with_cpu:
            from oracle.spectral_oracle import lambda_max_estimate
            import workloads as W
            w0 = Wm[0].cpu().numpy()
            v0 = W.splitmix_start_vectors(1, r, SPECTRAL_K)[0]
            t0 = time.perf_counter()
            lambda_max_estimate(w0, v0, SPECTRAL_ITERS)
            sec = time.perf_counter() - t0
            case["cpu_baseline"] = {"value": 1.0 / (sec * b), "unit": "calls/s", "cores": blas_threads(),
                                    "kind": "oracle",
                                    "sample": f"one {r}x{r} matrix of the stack (fp64 numpy), time x {b}"}
        out["cases"].append(case)
        del Wm
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--grads", type=int, default=3, help="distinct resident gradients cycled through")
    ap.add_argument("--no-sticky", action="store_true", help="retry the fp32 chain every step")
    ap.add_argument("--no-hint", action="store_true",
                    help="launch the fp32 chain every step even when every matrix is on the sticky fp64 chain")
    ap.add_argument("--chunks", type=int, default=0, help="concurrent chunks per stack (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time the eager steps only (default: also capture them as HIP graphs and time the replays, "
                         "which set the reported value)")
    ap.add_argument("--no-elementwise", action="store_true",
                    help="skip the AdamW / Lion measurement (the parameters Dion does not take)")
    ap.add_argument("--elementwise-only", action="store_true",
                    help="only the AdamW / Lion measurement, printed as one JSON line")
    ap.add_argument("--no-spectral", action="store_true",
                    help="skip the lambda_max estimate measurement (the spectral shift of the fallback)")
    ap.add_argument("--spectral-only", action="store_true",
                    help="only the lambda_max estimate measurement, printed as one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the Dion step here has no multi-GPU path.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import rank_orthonormalized_optimizer_amd as dion
    import workloads as W
    from rank_orthonormalized_optimizer_amd._lib import NUM_PHASES, PHASES
    from rank_orthonormalized_optimizer_amd.api import workspace_for

    dev = torch.device("cuda:0")
    if args.spectral_only:
        print(json.dumps(spectral_block(dev, torch.cuda.current_stream(dev), with_cpu=not args.no_cpu_baseline)),
              flush=True)
        return 0
    if args.elementwise_only:
        print(json.dumps(elementwise_block(dev, torch.cuda.current_stream(dev), with_cpu=not args.no_cpu_baseline)),
              flush=True)
        return 0
    wl = W.get(args.workload)
    print(f"[bench] workload {wl.name}: generating inputs", file=sys.stderr, flush=True)

    def dev_t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    stacks = []
    for gi, g in enumerate(wl.groups):
        X, M, Q = W.make_state(wl, gi)
        ngrad = 1 if wl.grad == "decaying_spectrum" else args.grads   # Haar factors cost seconds each
        grads = []
        for t in range(1, ngrad + 1):
            print(f"[bench] gradient {t}/{ngrad} of stack {gi}", file=sys.stderr, flush=True)
            grads.append(dev_t(W.make_grad(wl, gi, t)))
        stacks.append(dict(g=g, X=dev_t(X), M=dev_t(M), Q=dev_t(Q), G=grads,
                           flags=torch.zeros(g.batch, dtype=torch.int32, device=dev),
                           ws=workspace_for(g.m, g.n, g.batch, g.rank, dev)))
    opts = (0 if args.no_sticky else dion.OPT_STICKY_F64) | ((args.chunks & 15) << 8)
    stream = torch.cuda.current_stream(dev)
    for s in stacks:   # what DionStack does: skip launching the fp32 chain once a stack is all-fp64
        s["hint"] = None if (args.no_sticky or args.no_hint) else dion.StickyF64Hint(s["flags"])

    def one_step(k, events=None):
        for si, s in enumerate(stacks):
            g = s["g"]
            o = opts if s["hint"] is None else s["hint"].options(opts)
            dion.step_(s["X"], s["G"][k % len(s["G"])], s["M"], s["Q"], g.rank, wl.mu, wl.lr, wl.eps,
                       workspace=s["ws"], flags=s["flags"], options=o, stream=stream,
                       events=None if events is None else events[si])
            if s["hint"] is not None:
                s["hint"].after_step(stream)

    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 268435456 bytes read, 268435456 bytes written", file=sys.stderr, flush=True)
        del src, dst
    print("[bench] warmup", file=sys.stderr, flush=True)
    for k in range(args.warmup):
        one_step(k)
    torch.cuda.synchronize()

    # phase events for every call of the timed region (created by one record each beforehand)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(NUM_PHASES + 1)] for _ in stacks]
           for _ in range(args.steps)]
    for step_e in evs:
        for call_e in step_e:
            for e in call_e:
                e.record(stream)
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t0.record(stream)
    for k in range(args.steps):
        one_step(args.warmup + k, events=evs[k])
    t1.record(stream)
    enqueue = time.perf_counter() - w0
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    eager_ms = t0.elapsed_time(t1) / args.steps
    ms, launch, graph_ms = eager_ms, "eager", None
    if not args.eager:
        # The same steps captured once per resident gradient as HIP graphs and replayed: the
        # kernels and their arguments are those of the eager steps (options as the host hint has
        # settled them), so only the host's launch overhead between kernels goes away.
        ng = max(len(s_["G"]) for s_ in stacks)
        cap = torch.cuda.Stream(device=dev)
        cap.wait_stream(stream)
        graphs = []
        for j in range(ng):
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                gph.capture_begin()
                for s_ in stacks:
                    g_ = s_["g"]
                    o = opts if s_["hint"] is None else s_["hint"].options(opts)
                    dion.step_(s_["X"], s_["G"][j % len(s_["G"])], s_["M"], s_["Q"], g_.rank, wl.mu, wl.lr, wl.eps,
                               workspace=s_["ws"], flags=s_["flags"], options=o, stream=cap)
                gph.capture_end()
            graphs.append(gph)
        stream.wait_stream(cap)
        for k in range(2):
            graphs[(args.warmup + args.steps + k) % ng].replay()
        torch.cuda.synchronize()
        print(f"[bench] timing {args.steps} graph replays", file=sys.stderr, flush=True)
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for k in range(args.steps):
            graphs[(args.warmup + args.steps + 2 + k) % ng].replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        ms, launch = graph_ms, "hip_graph"
        del graphs

    # per-phase device times, averaged over the timed steps (summed over stacks)
    phase_ms = {p: 0.0 for p in PHASES}
    for step_e in evs:
        for call_e in step_e:
            for i, p in enumerate(PHASES):
                phase_ms[p] += call_e[i].elapsed_time(call_e[i + 1]) / args.steps
    n64 = int(sum(int((s["flags"] & dion.FLAG_F64).ne(0).sum()) for s in stacks))
    nbad = int(sum(int((s["flags"] & dion.FLAG_NONFINITE).ne(0).sum()) for s in stacks))
    nmat = sum(g.batch for g in wl.groups)

    # dominant single-kernel phase and its algorithmic flops per launch
    mnr64 = sum(int((s["flags"] & dion.FLAG_F64).ne(0).sum()) * s["g"].m * s["g"].n * s["g"].rank
                for s in stacks)
    mnr = sum(g.batch * g.m * g.n * g.rank for g in wl.groups)
    # The fp32 contractions run on the bf16 matrix cores as six bf16 products per fp32 product
    # (fp32-accurate split): their executed bf16 flops are SPLIT6 x the algorithmic fp32 flops and
    # are priced against the bf16 dense peak.
    SPLIT6 = 6.0
    kernels = {
        "f64_product": ("f64", 2.0 * mnr64, 1.0, "P0 = (M+G) Q, fp64 MFMA"),
        "f64_backproject": ("f64", 2.0 * mnr64, 1.0, "R = (M+G)^T P, fp64 MFMA"),
        "f32_product": ("bf16", 2.0 * (mnr - mnr64), SPLIT6, "P0 = (M+G) Q, fp32 as six bf16 MFMA products"),
        "f32_backproject": ("bf16", 2.0 * (mnr - mnr64), SPLIT6, "R = (M+G)^T P, fp32 as six bf16 MFMA products"),
        "update": ("bf16", 4.0 * mnr, SPLIT6, "P R^T and P Q'^T of the M, X update, fp32 as six bf16 MFMA products"),
    }
    dom = max(kernels, key=lambda k: phase_ms[k])
    dt_, alg_flops, factor, what = kernels[dom]
    flops = alg_flops * factor
    launches = len(stacks)
    secs = phase_ms[dom] * 1e-3
    achieved = flops / secs / 1e12 if secs > 0 else 0.0

    eff_gbs = algorithmic_bytes(wl) / (ms * 1e-3) / 1e9
    dtype = "f32" if n64 == 0 else ("f64+f32" if n64 == nmat else "f32|f64+f32")
    if wl.x_dtype == "bf16":
        dtype += " (bf16 X, G)"
    out = {
        "metric": "Dion updates/s and effective param GB/s (% HBM roofline) at rank frac 1/4",
        "value": 1000.0 / ms,
        "unit": "updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name,
                   "stacks": [f"{g.batch}x{g.m}x{g.n} r={g.rank}" for g in wl.groups],
                   "mu": wl.mu, "lr": wl.lr, "eps": wl.eps, "grad": wl.grad,
                   "sticky_fp64": not args.no_sticky,
                   "host_fp64_hint": not (args.no_sticky or args.no_hint), "chunks": args.chunks or "auto"},
        "effective_param_GBps": eff_gbs,
        "pct_hbm_roofline": 100.0 * eff_gbs / HBM_PEAK_GBS,
        "algorithmic_TFLOPs_per_s": algorithmic_flops(wl) / (ms * 1e-3) / 1e12,
        "matrices": nmat, "fp64_chain_matrices": n64, "nonfinite_matrices": nbad,
        "phase_ms": {k: round(v, 5) for k, v in phase_ms.items()},
        "launch": launch,
        "eager_ms_per_step": eager_ms,
        "graph_ms_per_step": graph_ms,
        "wall_s_timed_region_eager": wall,
        "host_enqueue_ms_per_step": 1000.0 * enqueue / args.steps,
        "roofline": {"bound": "mfma", "kernel": dom, "what": what, "dtype": dt_,
                     "achieved": achieved, "peak": PEAK_TFLOPS[dt_], "unit": "TFLOP/s",
                     "frac": achieved / PEAK_TFLOPS[dt_],
                     "flops_per_launch": flops / launches, "avg_launch_ms": phase_ms[dom] / launches,
                     "algorithmic_flops_per_launch": alg_flops / launches,
                     "algorithmic_TFLOPs_per_s": alg_flops / secs / 1e12 if secs > 0 else 0.0,
                     "mfma_flops_per_algorithmic_flop": factor,
                     "traffic": measured_traffic(wl.name, dom), "traffic_unit": "bytes/launch"},
    }
    if not args.no_elementwise:
        print("[bench] element-wise AdamW / Lion", file=sys.stderr, flush=True)
        out["elementwise"] = elementwise_block(dev, stream, with_cpu=not args.no_cpu_baseline)
    if not args.no_spectral:
        print("[bench] multi-power-iteration lambda_max estimate", file=sys.stderr, flush=True)
        out["spectral"] = spectral_block(dev, stream, with_cpu=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
