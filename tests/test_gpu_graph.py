"""The Dion step captured in a HIP graph and replayed gives bitwise the eager results.

bench.py times graph replays of the step, so this checks that capture changes nothing: the
same workload is stepped eagerly on one copy of the state and by replays of one captured step
on another (a fixed gradient buffer refilled before each replay), with eager torch work and
host synchronizations between the replays, and every replay is compared bit for bit with the
eager step it stands for.  Inputs: the reduced workloads (fp32 chain; fp64 chain with the
sticky flags).
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import to_numpy, to_torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wid,chunks", [(1, 1), (2, 1), (3, 1), (2, 3)])
def test_graph_replay_bitwise_equals_eager(cuda, wid, chunks):
    """chunks > 1 runs the stack on the library's internal streams (fork/join by events), which
    the capture records as parallel branches."""
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    from rank_orthonormalized_optimizer_amd._lib import opt_chunks
    wl = W.SMALL[wid]
    g = wl.groups[0]
    X, M, Q = W.make_state(wl, 0)
    grads = [to_torch(W.make_grad(wl, 0, t), cuda) for t in range(1, 5)]
    opts = dion.OPT_STICKY_F64 | opt_chunks(chunks)

    def state():
        return (to_torch(X, cuda), to_torch(M, cuda), to_torch(Q, cuda),
                torch.zeros(g.batch, dtype=torch.int32, device=cuda), dion.api.workspace_for(g.m, g.n, g.batch,
                                                                                           g.rank, cuda))
    Xa, Ma, Qa, Fa, Wa = state()
    Xb, Mb, Qb, Fb, Wb = state()
    stream = torch.cuda.current_stream(cuda)
    # step 1 eagerly on both (sets the sticky flags)
    for (x, m, q, f, w) in ((Xa, Ma, Qa, Fa, Wa), (Xb, Mb, Qb, Fb, Wb)):
        dion.step_(x, grads[0], m, q, g.rank, wl.mu, wl.lr, wl.eps, workspace=w, flags=f, options=opts)
    torch.cuda.synchronize()
    gbuf = grads[1].clone()
    cap = torch.cuda.Stream(device=cuda)
    cap.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    print(f"[graph] {wl.name}: capture", flush=True)
    with torch.cuda.stream(cap):
        graph.capture_begin()
        dion.step_(Xb, gbuf, Mb, Qb, g.rank, wl.mu, wl.lr, wl.eps, workspace=Wb, flags=Fb, options=opts,
                   stream=cap)
        graph.capture_end()
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    for t in (1, 2, 3):
        print(f"[graph] {wl.name}: step {t + 1}", flush=True)
        dion.step_(Xa, grads[t], Ma, Qa, g.rank, wl.mu, wl.lr, wl.eps, workspace=Wa, flags=Fa, options=opts)
        gbuf.copy_(grads[t])
        junk = (Xa.float() * 2).sum()   # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for a, b in ((Xa, Xb), (Ma, Mb), (Qa, Qb), (Fa, Fb)):
            assert np.array_equal(to_numpy(a), to_numpy(b)), (wid, t)


def test_graphed_step_api(cuda):
    """api.GraphedStep: a DionStack step captured once and replayed with a refilled gradient buffer
    equals the DionStack's eager steps bit for bit."""
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    wl = W.SMALL[2]
    g = wl.groups[0]
    X, _, _ = W.make_state(wl, 0)
    grads = [to_torch(W.make_grad(wl, 0, t), cuda) for t in range(1, 5)]
    sa = dion.DionStack(g.batch, g.m, g.n, rank=g.rank, mu=wl.mu, lr=wl.lr, eps=wl.eps, device=cuda)
    sb = dion.DionStack(g.batch, g.m, g.n, rank=g.rank, mu=wl.mu, lr=wl.lr, eps=wl.eps, device=cuda)
    Xa, Xb = to_torch(X, cuda), to_torch(X, cuda)
    for t in (0, 1):   # two eager steps on both: flags and the host hint settle
        sa.step(Xa, grads[t])
        sb.step(Xb, grads[t])
    torch.cuda.synchronize()
    gbuf = grads[2].clone()
    gs = dion.GraphedStep(sb, Xb, gbuf)
    for t in (2, 3):
        print(f"[graph] GraphedStep step {t + 1}", flush=True)
        sa.step(Xa, grads[t])
        gbuf.copy_(grads[t])
        gs.replay()
        torch.cuda.synchronize()
        for a, b in ((Xa, Xb), (sa.M, sb.M), (sa.Q, sb.Q), (sa.flags, sb.flags)):
            assert np.array_equal(to_numpy(a), to_numpy(b)), t
