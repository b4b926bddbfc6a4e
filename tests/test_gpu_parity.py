"""GPU parity: the HIP step against the fp64 oracle, teacher-forced, per step.

Reduced-size versions of the five workloads (same recipes, shapes spanning
several 64-wide tiles with ragged tails) are compared element by element
through P Q^T, M and X, to 1e-4 relative Frobenius error for fp32 weights and
2e-2 for bf16 weights.
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import compare_step, to_numpy, to_torch, tol_for

pytestmark = pytest.mark.gpu


def run_teacher_forced(wl, device, options=0, steps=None):
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    report = []
    for gi, g in enumerate(wl.groups):
        X, M, Q = W.make_state(wl, gi)
        Xd, Md, Qd = to_torch(X, device), to_torch(M, device), to_torch(Q, device)
        flags = torch.zeros(g.batch, dtype=torch.int32, device=device)
        ws = dion.api.workspace_for(g.m, g.n, g.batch, g.rank, device)
        for t in range(1, (steps or wl.steps) + 1):
            G = W.make_grad(wl, gi, t)
            Gd = to_torch(G, device)
            pre = {"X": to_numpy(Xd), "M": to_numpy(Md), "Q": to_numpy(Qd)}
            print(f"[parity] {wl.name} group {gi} {g} step {t}", flush=True)
            dion.step_(Xd, Gd, Md, Qd, g.rank, wl.mu, wl.lr, wl.eps, workspace=ws, flags=flags, options=options)
            torch.cuda.synchronize()
            P = ws[:4 * g.batch * g.m * g.rank].view(torch.float32).view(g.batch, g.m, g.rank)
            post = {"X": to_numpy(Xd), "M": to_numpy(Md), "Q": to_numpy(Qd), "P": to_numpy(P)}
            errs = compare_step(wl, pre, post, G, g.rank)
            report.append((gi, t, errs, to_numpy(flags)))
    return report


def check(report, tol):
    worst = {}
    for gi, t, errs, flags in report:
        for i, e in enumerate(errs):
            assert not (flags[i] & 2), f"group {gi} step {t} matrix {i}: non-finite flag"
            for k in ("PQ", "M", "X"):
                if k in e:
                    worst[k] = max(worst.get(k, 0.0), e[k])
                    assert e[k] <= tol, f"group {gi} step {t} matrix {i}: {k} rel err {e[k]:.3e} > {tol}"
            if "orth" in e:
                assert e["orth"] <= 1e-4, f"group {gi} step {t} matrix {i}: |P^T P - I| = {e['orth']:.3e}"
    print("worst", worst, flush=True)
    return worst


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_small_workloads_teacher_forced(cuda, wid):
    wl = W.SMALL[wid]
    check(run_teacher_forced(wl, cuda), tol_for(wl))


@pytest.mark.parametrize("wid", [1, 3])
def test_forced_fp64_chain(cuda, wid):
    import rank_orthonormalized_optimizer_amd as dion
    wl = W.SMALL[wid]
    rep = run_teacher_forced(wl, cuda, options=dion.OPT_FORCE_F64, steps=2)
    for _, _, _, flags in rep:
        assert np.all(flags & dion.FLAG_F64)
    check(rep, tol_for(wl))


def test_fallback_fires_on_ill_conditioned(cuda):
    """The low-rank-plus-noise gradients make P0 ill-conditioned: every matrix must take the fp64 chain."""
    import rank_orthonormalized_optimizer_amd as dion
    wl = W.SMALL[2]
    rep = run_teacher_forced(wl, cuda, steps=2)
    for _, _, _, flags in rep:
        assert np.all(flags & dion.FLAG_F64), flags
    check(rep, tol_for(wl))


@pytest.mark.parametrize("recipe,options", [("gauss", 0), ("lowrank_noise", "f64")])
def test_many_rank_blocks(cuda, recipe, options):
    """r = 330: six 64-wide Cholesky blocks with a ragged last one, three inverse-doubling levels."""
    import rank_orthonormalized_optimizer_amd as dion
    base = W.SMALL[1] if recipe == "gauss" else W.SMALL[2]
    wl = base.with_groups(W.Group(2, 520, 400, 330), name=f"blocks-{recipe}", steps=2)
    opts = dion.OPT_FORCE_F64 if options == "f64" else 0
    rep = run_teacher_forced(wl, cuda, options=opts)
    check(rep, tol_for(wl))


def test_chunking_is_bitwise_invariant(cuda):
    """Splitting the stack into concurrent chunks changes nothing: matrices are independent."""
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    from rank_orthonormalized_optimizer_amd._lib import opt_chunks
    wl = W.SMALL[2].with_groups(W.Group(5, 320, 288, 72), name="chunks")
    X, M, Q = W.make_state(wl, 0)
    outs = []
    for nc in (1, 2, 3, 5):
        Xd, Md, Qd = to_torch(X, cuda), to_torch(M, cuda), to_torch(Q, cuda)
        flags = torch.zeros(5, dtype=torch.int32, device=cuda)
        for t in (1, 2):
            Gd = to_torch(W.make_grad(wl, 0, t), cuda)
            dion.step_(Xd, Gd, Md, Qd, 72, wl.mu, wl.lr, wl.eps, flags=flags,
                       options=dion.OPT_STICKY_F64 | opt_chunks(nc))
        torch.cuda.synchronize()
        outs.append((to_numpy(Xd), to_numpy(Md), to_numpy(Qd), to_numpy(flags)))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
