"""dion_step_batched_noalloc: the Dion step with the library's built-in scratch instead of a
caller workspace, for callers that cannot allocate.  Through the C ABI, its results must equal
those of dion_step_batched on the same inputs bit for bit (same kernels, same arithmetic; the
step does not depend on its scratch's contents on entry), on two calls in a row, the second on
a smaller stack, so the second runs over scratch the first left behind.  The host-side
rejections need no GPU."""
import numpy as np
import pytest

import workloads as W
from rank_orthonormalized_optimizer_amd import _lib
from tests.harness import to_numpy, to_torch

DT = {"f32": _lib.F32, "bf16": _lib.BF16}


def _call_noalloc(m=64, n=96, batch=2, rank=8, options=0, X=0, G=0, M=0, Q=0):
    return _lib.step_batched_noalloc_raw(X, G, M, Q, m, n, batch, rank, 0.95, 0.01, 1e-8, _lib.F32, _lib.F32, 0,
                                         options, 0)


def test_noalloc_rejects_stacks_beyond_its_scratch():
    # 24 x 1024^2 at r = 256 needs about 283 MiB of scratch: rejected on the host, before any pointer check
    assert _lib.workspace_size(1024, 1024, 24, 256) > _lib.NOALLOC_SCRATCH_BYTES
    assert _call_noalloc(1024, 1024, 24, 256) == _lib.ERR_SCRATCH
    assert "scratch" in _lib.strerror(_lib.ERR_SCRATCH)
    # the largest of a family that still fits is not rejected for its size (only for its null pointers)
    assert _lib.workspace_size(1024, 1024, 4, 256) <= _lib.NOALLOC_SCRATCH_BYTES
    assert _call_noalloc(1024, 1024, 4, 256) == _lib.ERR_NULL
    # one chunk only; the other argument checks are those of dion_step_batched
    assert _call_noalloc(options=_lib.opt_chunks(2)) == _lib.ERR_OPTION
    assert _call_noalloc(options=_lib.opt_chunks(1)) == _lib.ERR_NULL
    assert _call_noalloc(rank=97) == _lib.ERR_RANK
    assert _call_noalloc(batch=0) == _lib.OK


def _pair(wl, gi, device, options):
    """One step of stack gi through both entry points on identical copies of the inputs."""
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    g = wl.groups[gi]
    X, M, Q = W.make_state(wl, gi)
    M[:] = W.store(1e-3 * np.random.default_rng(gi + 11).standard_normal(M.shape), "f32")
    G = W.make_grad(wl, gi, 1)
    outs = []
    for which in ("workspace", "noalloc"):
        Xd, Md, Qd, Gd = to_torch(X, device), to_torch(M, device), to_torch(Q, device), to_torch(G, device)
        flags = torch.zeros(g.batch, dtype=torch.int32, device=device)
        stream = int(torch.cuda.current_stream(device).cuda_stream)
        args = (Xd.data_ptr(), Gd.data_ptr(), Md.data_ptr(), Qd.data_ptr(), g.m, g.n, g.batch, g.rank,
                wl.mu, wl.lr, wl.eps, DT[wl.x_dtype], DT[wl.g_dtype])
        print(f"[noalloc] {wl.name} {g} via {which}", flush=True)
        if which == "workspace":
            ws = dion.api.workspace_for(g.m, g.n, g.batch, g.rank, device)
            st = _lib.step_batched_raw(*args, ws.data_ptr(), ws.numel(), flags.data_ptr(), options, stream)
        else:
            st = _lib.step_batched_noalloc_raw(*args, flags.data_ptr(), options, stream)
        assert st == _lib.OK, _lib.strerror(st)
        torch.cuda.synchronize()
        outs.append([to_numpy(t) for t in (Xd, Md, Qd, flags)])
    return outs


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry(cuda):
    import rank_orthonormalized_optimizer_amd as dion
    # call 1: an ill-conditioned fp32 stack (the fp64 chain, 3 x 320 x 288, r = 72)
    # call 2: a smaller bf16 pair of stacks' first stack (2 x 200 x 136, r = 17) on the fp32 chain
    calls = [(W.SMALL[2], 0, dion.OPT_STICKY_F64), (W.SMALL[3], 0, 0)]
    sizes = [_lib.workspace_size(c[0].groups[c[1]].m, c[0].groups[c[1]].n, c[0].groups[c[1]].batch,
                                 c[0].groups[c[1]].rank) for c in calls]
    assert sizes[1] < sizes[0] <= _lib.NOALLOC_SCRATCH_BYTES
    for wl, gi, opts in calls:
        ref, got = _pair(wl, gi, cuda, opts)
        for name, a, b in zip(("X", "M", "Q", "flags"), ref, got):
            assert a.dtype == b.dtype and a.shape == b.shape
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{wl.name}: {name} differs"
        assert not np.any(got[3] & _lib.FLAG_NONFINITE)
