"""Race detection by bitwise repeat: independent stacks stepped concurrently, each on its own
stream (their kernels then share the CUs and run out of their usual lockstep), must give the
same bits as the same steps run one stack after another on one stream.  The shapes take the
weight pass's large-tile branch-free path and the split-bf16 products' branch-free staging,
with fp32 and bf16 weights."""
import numpy as np
import pytest

import workloads as W
from tests.harness import to_numpy, to_torch

pytestmark = pytest.mark.gpu

STACKS = [
    W.SMALL[1].with_groups(W.Group(12, 512, 512, 64), name="conc-f32-a"),
    W.SMALL[1].with_groups(W.Group(8, 384, 640, 96), name="conc-f32-b"),
    W.SMALL[3].with_groups(W.Group(12, 512, 512, 64), name="conc-bf16"),
    W.SMALL[2].with_groups(W.Group(6, 256, 256, 64), name="conc-f64-chain"),
]


def _run(device, concurrent: bool, steps: int = 3):
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    state = []
    for wl in STACKS:
        g = wl.groups[0]
        X, M, Q = W.make_state(wl, 0)
        state.append(dict(wl=wl, g=g, X=to_torch(X, device), M=to_torch(M, device), Q=to_torch(Q, device),
                          G=[to_torch(W.make_grad(wl, 0, t), device) for t in range(1, steps + 1)],
                          flags=torch.zeros(g.batch, dtype=torch.int32, device=device),
                          ws=dion.api.workspace_for(g.m, g.n, g.batch, g.rank, device)))
    torch.cuda.synchronize()
    base = torch.cuda.current_stream(device)
    side = [torch.cuda.Stream(device=device) for _ in state]
    for t in range(steps):
        fork = torch.cuda.Event()
        fork.record(base)
        for s, st in zip(state, side):
            stream = base
            if concurrent:
                st.wait_event(fork)
                stream = st
            wl, g = s["wl"], s["g"]
            dion.step_(s["X"], s["G"][t], s["M"], s["Q"], g.rank, wl.mu, wl.lr, wl.eps, workspace=s["ws"],
                       flags=s["flags"], options=dion.OPT_STICKY_F64, stream=stream)
        if concurrent:
            for st in side:
                base.wait_stream(st)
    torch.cuda.synchronize()
    return [[to_numpy(s[k]) for k in ("X", "M", "Q", "flags")] for s in state]


def test_concurrent_stacks_are_bitwise_serial(cuda):
    print("[concurrency] serial", flush=True)
    ref = _run(cuda, concurrent=False)
    for rep in range(3):
        print(f"[concurrency] concurrent, repeat {rep}", flush=True)
        got = _run(cuda, concurrent=True)
        for wl, a, b in zip(STACKS, ref, got):
            for name, x, y in zip(("X", "M", "Q", "flags"), a, b):
                assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{wl.name}: {name} differs (repeat {rep})"
