#!/usr/bin/env python3
"""Benchmark of the Dion step on one MI355X.

A "step" is one Dion update of every matrix of a workload (all its stacks), with the
inputs already resident in HBM.  The headline workload is the rank-fraction-1/4
attention stack: 24 fp32 matrices of 1024 x 1024 at r = 256 with low-rank-plus-noise
gradients (see workloads/).  The default run also measures every other workload and
reports them in a "configs" array.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload 1..5] [--configs 1,2,3,4,5 | none]
                  [--no-cpu-baseline] [--eager]

Inputs are drawn on the device with the workloads' recipes (workloads.make_state_device and
make_grad_device: same distributions as the host generators the parity tests use, drawn by a
seeded torch generator); --host-inputs draws them on the host instead.

Per workload the K timed steps run twice: eagerly (one host launch per kernel, with the
library's phase events) and as replays of the same steps captured in HIP graphs (one graph per
resident gradient).  The replays set the value; both times are reported ("eager_ms_per_step",
"graph_ms_per_step"), and --eager times the eager steps only.

Metric: updates/s (steps per second over the whole workload), with the effective parameter
bandwidth (algorithmic bytes / step time) and its share of the 8 TB/s HBM peak alongside.
Every phase of the step is priced against the roofline that bounds it ("phase_roofline"; the
phase times come from HIP events the library records at its phase boundaries, on the stream
the kernels run on), the dominant single-kernel phase is the "roofline" entry, and the
multi-kernel QR phase has its own "qr_roofline".  "cpu_baseline" times the fp64 oracle on
the host cores over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"f64": 78.6, "f32": 157.3, "bf16": 2500.0}
METRIC = "Dion updates/s and effective param GB/s (% HBM roofline) at rank frac 1/4"
HEADLINE = 2


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


def blas_info() -> dict:
    """BLAS vendor, version and thread count numpy runs on (threadpoolctl), with the host's CPU."""
    info = {"cpu_count": os.cpu_count(), "cpu_model": platform.processor() or None}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = int(max(d.get("num_threads", 0) for d in blas))
    except Exception:
        pass
    info.setdefault("blas_threads", os.cpu_count() or 1)
    return info


def blas_threads() -> int:
    return int(blas_info()["blas_threads"])


def cpu_baseline(wl, samples, budget_s: float) -> dict:
    """The fp64 oracle as it stands, on the host cores, over a bounded sample of the workload.

    ``samples``: per stack, the step-1 inputs (X, G, M, Q as host arrays) of its first matrix.
    Each stack's matrix is stepped while its share of the budget lasts (at least once); the
    mean time per matrix is scaled to the stack size and summed over the stacks.
    """
    import numpy as np

    import workloads as W
    from oracle import dion_step
    t_all = time.perf_counter()
    per_group = []
    for (g, (X, G, M, Q)) in zip(wl.groups, samples):
        args = (W.to_f64(X, wl.x_dtype), W.to_f64(G, wl.g_dtype), M.astype(np.float64), Q.astype(np.float64))
        share = budget_s / len(wl.groups)
        times, t0 = [], time.perf_counter()
        while not times or time.perf_counter() - t0 < share:
            t1 = time.perf_counter()
            dion_step(*args, wl.mu, wl.lr, wl.eps)
            times.append(time.perf_counter() - t1)
        per_group.append((g, float(np.mean(times)), len(times)))
    step_s = sum(g.batch * t for g, t, _ in per_group)
    sample = "; ".join(f"{k} steps of one matrix of the {g.batch}x{g.m}x{g.n} r={g.rank} stack"
                       for g, _, k in per_group)
    info = blas_info()
    return {"value": 1.0 / step_s, "unit": "updates/s", "cores": info["blas_threads"], "kind": "oracle",
            "sample": sample + f" (step-1 inputs, fp64 numpy; mean time per matrix x stack size; "
                               f"{time.perf_counter() - t_all:.1f} s of CPU work)",
            "s_per_step": step_s, "host": info}


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
                "roofline": {"bound": "mfma", "dtype": "f64", "kernel": "mpi_product_kernel", "achieved": tf,
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


SPLIT6 = 6.0   # bf16 MFMA products per fp32 product in the exact split form the fp32 contractions use
SPLIT2 = 3.0   # bf16 MFMA products per fp32 product of the weight pass (two-part split: hh, hl, lh)


def phase_rooflines(wl, stacks, phase_ms, dion) -> dict:
    """Every phase of the step against the roofline that bounds it.  ``phase_ms``: device time
    per step of each phase, summed over the stacks; the flops and bytes are algorithmic and
    counted for the matrices each chain actually owned (flags after the last timed step)."""
    f64m = [int((s["flags"] & dion.FLAG_F64).ne(0).sum()) for s in stacks]
    # bf16 weights run the three big contractions as plain bf16 products (one MFMA product per
    # algorithmic one); fp32 weights as the exact six-product split
    split = 1.0 if wl.x_dtype == "bf16" else SPLIT6
    how = "plain bf16 MFMA products" if split == 1.0 else "fp32 as six bf16 MFMA products"
    # the weight pass of fp32 weights keeps three part products (its operands are final)
    usplit = 1.0 if wl.x_dtype == "bf16" else SPLIT2
    uhow = "plain bf16 MFMA products" if usplit == 1.0 else "fp32 as three bf16 part products (two-part split)"
    out = {}

    def add(name, kind, amount, peak_key, factor=1.0, what=""):
        ms = phase_ms[name]
        secs = ms * 1e-3
        ent = {"ms": ms, "what": what}
        if kind == "flops":
            exe = amount * factor
            ach = exe / secs / 1e12 if secs > 0 and amount > 0 else 0.0
            ent.update({"bound": "mfma", "dtype": peak_key, "algorithmic_flops": amount,
                        "executed_flops": exe, "achieved": ach, "peak": PEAK_TFLOPS[peak_key], "unit": "TFLOP/s",
                        "frac": ach / PEAK_TFLOPS[peak_key]})
        else:
            ach = amount / secs / 1e9 if secs > 0 and amount > 0 else 0.0
            ent.update({"bound": "hbm", "algorithmic_bytes": amount, "achieved": ach, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": ach / HBM_PEAK_GBS})
        out[name] = ent

    mnr32 = mnr64 = qr32 = qr64 = nb = ub = 0.0
    for s, k64 in zip(stacks, f64m):
        g = s["g"]
        m, n, r, b = g.m, g.n, g.rank, g.batch
        k32 = b - k64
        mnr32 += k32 * m * n * r
        mnr64 += k64 * m * n * r
        qrf = 6.0 * m * r * r + 2.0 * r ** 3 / 3.0
        qr32 += k32 * qrf
        qr64 += k64 * qrf
        nb += k32 * n * r * 8.0 + k64 * (n * r * 16.0 + m * r * 12.0)
        bx = 2 if wl.x_dtype == "bf16" else 4
        ub += b * (m * n * (bx + 8 + 2 * bx) + 4.0 * (m + 2 * n) * r)
    add("f32_product", "flops", 2.0 * mnr32, "bf16", split, "P0 = (M+G) Q, " + how)
    add("f32_qr", "flops", qr32, "f32", 1.0, "CholeskyQR2 of the fp32 chain, 6 m r^2 + 2 r^3 / 3 per matrix")
    add("f32_backproject", "flops", 2.0 * mnr32, "bf16", split, "R = (M+G)^T P, " + how)
    add("f64_product", "flops", 2.0 * mnr64, "f64", 1.0, "P0 = (M+G) Q, fp64 MFMA")
    add("f64_qr", "flops", qr64, "f64", 1.0, "CholeskyQR2 (shifted CholeskyQR3) of the fp64 chain, "
                                             "6 m r^2 + 2 r^3 / 3 per matrix")
    add("f64_backproject", "flops", 2.0 * mnr64, "f64", 1.0, "R = (M+G)^T P, fp64 MFMA")
    add("norms", "bytes", nb, "hbm", 1.0, "column norms of R, Q' = R c; fp64-chain P, R rounded to fp32")
    add("update", "flops", 4.0 * (mnr32 + mnr64), "bf16", usplit, "P R^T and P Q'^T of the M, X update, " + uhow)
    for k in ("f32_product", "f32_backproject"):   # the HBM side of the products: B read once
        bg = sum(s_["g"].batch * s_["g"].m * s_["g"].n for s_ in stacks) * (4 + (2 if wl.g_dtype == "bf16" else 4))
        if k.startswith("f32") and f64m and sum(f64m) == sum(s_["g"].batch for s_ in stacks):
            bg = 0.0
        ms = phase_ms[k]
        ach = bg / (ms * 1e-3) / 1e9 if ms > 0 and bg > 0 else 0.0
        out[k]["hbm"] = {"algorithmic_bytes": bg, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS}
    out["update"]["hbm"] = {"algorithmic_bytes": ub,
                            "achieved": ub / (phase_ms["update"] * 1e-3) / 1e9 if phase_ms["update"] > 0 else 0.0,
                            "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    out["update"]["hbm"]["frac"] = out["update"]["hbm"]["achieved"] / HBM_PEAK_GBS
    return out


def measure(wl, dev, stream, args, cpu_s: float, host_inputs: bool) -> dict:
    """Time one workload: W warm-up steps, K eager steps with phase events, K graph replays."""
    import numpy as np
    import torch

    import rank_orthonormalized_optimizer_amd as dion
    import workloads as W
    from rank_orthonormalized_optimizer_amd._lib import NUM_PHASES, PHASES
    from rank_orthonormalized_optimizer_amd.api import workspace_for
    from tests.harness import to_numpy, to_torch

    print(f"[bench] workload {wl.name}: inputs", file=sys.stderr, flush=True)
    stacks, samples = [], []
    for gi, g in enumerate(wl.groups):
        ngrad = 1 if wl.grad == "decaying_spectrum" else args.grads
        if host_inputs:
            X, M, Q = (to_torch(a, dev) for a in W.make_state(wl, gi))
            grads = [to_torch(W.make_grad(wl, gi, t), dev) for t in range(1, ngrad + 1)]
        else:
            X, M, Q = W.make_state_device(wl, gi, dev)
            grads = [W.make_grad_device(wl, gi, t, dev) for t in range(1, ngrad + 1)]
        samples.append((to_numpy(X[0]), to_numpy(grads[0][0]), to_numpy(M[0]), to_numpy(Q[0])))
        stacks.append(dict(g=g, X=X, M=M, Q=Q, G=grads, flags=torch.zeros(g.batch, dtype=torch.int32, device=dev),
                           ws=workspace_for(g.m, g.n, g.batch, g.rank, dev)))
    torch.cuda.synchronize()
    opts = (0 if args.no_sticky else dion.OPT_STICKY_F64) | ((args.chunks & 15) << 8)
    for s in stacks:   # what DionStack does: skip launching the fp32 chain once a stack is all-fp64
        s["hint"] = None if (args.no_sticky or args.no_hint) else dion.StickyF64Hint(s["flags"])

    # independent stacks run concurrently, each on its own stream forked from and joined back
    # into the launch stream, so one stack's latency-bound QR overlaps another's streaming passes
    side = [torch.cuda.Stream(device=dev) for _ in stacks] if len(stacks) > 1 and not args.serial_stacks else None

    def issue(k, base, events=None, hints=True):
        if side is not None:
            fork = torch.cuda.Event()
            fork.record(base)
        for si, s in enumerate(stacks):
            g = s["g"]
            st = base if side is None else side[si]
            if side is not None:
                st.wait_event(fork)
            o = opts if s["hint"] is None else s["hint"].options(opts)
            dion.step_(s["X"], s["G"][k % len(s["G"])], s["M"], s["Q"], g.rank, wl.mu, wl.lr, wl.eps,
                       workspace=s["ws"], flags=s["flags"], options=o, stream=st,
                       events=None if events is None else events[si])
            if hints and s["hint"] is not None:
                s["hint"].after_step(st)
        if side is not None:
            for st in side:
                base.wait_stream(st)

    def one_step(k, events=None):
        issue(k, stream, events)

    print(f"[bench] {wl.name}: warmup", file=sys.stderr, flush=True)
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
    print(f"[bench] {wl.name}: timing {args.steps} steps", file=sys.stderr, flush=True)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
                issue(j, cap, hints=False)
                gph.capture_end()
            graphs.append(gph)
        stream.wait_stream(cap)
        for k in range(2):
            graphs[(args.warmup + args.steps + k) % ng].replay()
        torch.cuda.synchronize()
        print(f"[bench] {wl.name}: timing {args.steps} graph replays", file=sys.stderr, flush=True)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
    nsh = int(sum(int((s["flags"] & dion.FLAG_SHIFTED).ne(0).sum()) for s in stacks))
    nhh = int(sum(int((s["flags"] & dion.FLAG_HOUSEHOLDER).ne(0).sum()) for s in stacks))
    nmat = sum(g.batch for g in wl.groups)
    pr = phase_rooflines(wl, stacks, phase_ms, dion)
    single = ("f32_product", "f32_backproject", "f64_product", "f64_backproject", "update")
    dom = max(single, key=lambda k: phase_ms[k])
    d = pr[dom]
    launches = len(stacks)
    roof = {"bound": d["bound"], "kernel": dom, "what": d["what"], "dtype": d["dtype"],
            "achieved": d["achieved"], "peak": d["peak"], "unit": d["unit"], "frac": d["frac"],
            "flops_per_launch": d["executed_flops"] / launches, "avg_launch_ms": phase_ms[dom] / launches,
            "algorithmic_flops_per_launch": d["algorithmic_flops"] / launches,
            "algorithmic_TFLOPs_per_s": (d["algorithmic_flops"] / (phase_ms[dom] * 1e-3) / 1e12
                                         if phase_ms[dom] > 0 else 0.0),
            "mfma_flops_per_algorithmic_flop": d["executed_flops"] / d["algorithmic_flops"]
            if d["algorithmic_flops"] else None,
            "traffic": measured_traffic(wl.name, dom), "traffic_unit": "bytes/launch"}
    qr = pr["f64_qr"] if phase_ms["f64_qr"] >= phase_ms["f32_qr"] else pr["f32_qr"]
    eff_gbs = algorithmic_bytes(wl) / (ms * 1e-3) / 1e9
    dtype = "f32" if n64 == 0 else ("f64+f32" if n64 == nmat else "f32|f64+f32")
    if wl.x_dtype == "bf16":
        dtype = "bf16 products, f32 QR (bf16 X, G; f32 M, Q)" if n64 == 0 else dtype + " (bf16 X, G)"
    ent = {
        "workload": wl.name,
        "stacks": [f"{g.batch}x{g.m}x{g.n} r={g.rank}" for g in wl.groups],
        "mu": wl.mu, "lr": wl.lr, "eps": wl.eps, "grad": wl.grad,
        "inputs": "host generators" if host_inputs else "device generators (same recipes)",
        "value": 1000.0 / ms, "unit": "updates/s", "ms_per_step": ms, "dtype": dtype,
        "effective_param_GBps": eff_gbs, "pct_hbm_roofline": 100.0 * eff_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": algorithmic_bytes(wl),
        "algorithmic_flops_per_step": algorithmic_flops(wl),
        "algorithmic_TFLOPs_per_s": algorithmic_flops(wl) / (ms * 1e-3) / 1e12,
        "params": wl.params(), "matrices": nmat, "fp64_chain_matrices": n64, "shifted_matrices": nsh,
        "householder_matrices": nhh, "nonfinite_matrices": nbad,
        "phase_ms": {k: round(v, 5) for k, v in phase_ms.items()},
        "phase_roofline": pr,
        "concurrent_stacks": side is not None,
        "launch": launch, "eager_ms_per_step": eager_ms, "graph_ms_per_step": graph_ms,
        "wall_s_timed_region_eager": wall, "host_enqueue_ms_per_step": 1000.0 * enqueue / args.steps,
        "roofline": roof,
        "qr_roofline": {k: qr[k] for k in ("bound", "dtype", "achieved", "peak", "unit", "frac", "ms",
                                           "algorithmic_flops", "what")},
    }
    del stacks
    torch.cuda.empty_cache()
    if cpu_s > 0:
        print(f"[bench] {wl.name}: cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        ent["cpu_baseline"] = cpu_baseline(wl, samples, cpu_s)
    return ent


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=HEADLINE, choices=[1, 2, 3, 4, 5],
                    help="the headline workload (default: the rank-fraction-1/4 attention stack)")
    ap.add_argument("--configs", default="1,2,3,4,5",
                    help="workloads also measured into the 'configs' array ('none' to skip)")
    ap.add_argument("--host-inputs", action="store_true", help="draw inputs with the host generators")
    ap.add_argument("--grads", type=int, default=3, help="distinct resident gradients cycled through")
    ap.add_argument("--no-sticky", action="store_true", help="retry the fp32 chain every step")
    ap.add_argument("--no-hint", action="store_true",
                    help="launch the fp32 chain every step even when every matrix is on the sticky fp64 chain")
    ap.add_argument("--chunks", type=int, default=0, help="concurrent chunks per stack (0 = library default)")
    ap.add_argument("--serial-stacks", action="store_true",
                    help="step a workload's stacks one after another on one stream (default: concurrently)")
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
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle budget of the headline workload")
    ap.add_argument("--config-cpu-seconds", type=float, default=4.0, help="oracle budget of each other workload")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the Dion step here has no multi-GPU path.", file=sys.stderr)
        return 2

    import torch

    import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.spectral_only:
        print(json.dumps(spectral_block(dev, stream, with_cpu=not args.no_cpu_baseline)), flush=True)
        return 0
    if args.elementwise_only:
        print(json.dumps(elementwise_block(dev, stream, with_cpu=not args.no_cpu_baseline)), flush=True)
        return 0
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 268435456 bytes read, 268435456 bytes written", file=sys.stderr, flush=True)
        del src, dst
    cpu = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    head = measure(W.get(args.workload), dev, stream, args, cpu, args.host_inputs)
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {"workload": head["workload"], "stacks": head["stacks"], "mu": head["mu"], "lr": head["lr"],
                   "eps": head["eps"], "grad": head["grad"], "inputs": head["inputs"],
                   "sticky_fp64": not args.no_sticky, "host_fp64_hint": not (args.no_sticky or args.no_hint),
                   "chunks": args.chunks or "auto"},
    }
    for k in ("effective_param_GBps", "pct_hbm_roofline", "algorithmic_TFLOPs_per_s", "matrices",
              "fp64_chain_matrices", "shifted_matrices", "householder_matrices", "nonfinite_matrices", "phase_ms",
              "phase_roofline", "launch", "eager_ms_per_step", "graph_ms_per_step", "wall_s_timed_region_eager",
              "host_enqueue_ms_per_step", "roofline", "qr_roofline"):
        out[k] = head[k]
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    if args.configs != "none":
        out["configs"] = []
        for wid in [int(x) for x in args.configs.split(",") if x.strip()]:
            if wid == args.workload:
                ent = dict(head)
            else:
                ccpu = 0.0 if args.no_cpu_baseline else args.config_cpu_seconds
                ent = measure(W.get(wid), dev, stream, args, ccpu, args.host_inputs)
            ent["wid"] = wid
            out["configs"].append(ent)
    if not args.no_elementwise:
        print("[bench] element-wise AdamW / Lion", file=sys.stderr, flush=True)
        out["elementwise"] = elementwise_block(dev, stream, with_cpu=not args.no_cpu_baseline)
    if not args.no_spectral:
        print("[bench] multi-power-iteration lambda_max estimate", file=sys.stderr, flush=True)
        out["spectral"] = spectral_block(dev, stream, with_cpu=not args.no_cpu_baseline)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
