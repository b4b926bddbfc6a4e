"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

The oracle recomputes sampled matrices of every stack one by one (teacher-forced:
from the exact pre-step state bits the GPU used); properties that hold at any
size are checked on every matrix on the GPU in fp64 (torch used as a checker only):
  * P^T P = I for the orthonormal factor left in the workspace,
  * full rank (r = min(m, n)): M' = mu B exactly in exact arithmetic,
  * no matrix flagged non-finite.
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import compare_step, to_numpy, to_torch, tol_for

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _run(wl, device, steps, sample):
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    out = []
    for gi, g in enumerate(wl.groups):
        print(f"[fullsize] {wl.name} group {gi} {g}: inputs", flush=True)
        X, M, Q = W.make_state(wl, gi)
        Xd, Md, Qd = to_torch(X, device), to_torch(M, device), to_torch(Q, device)
        del X, M, Q
        flags = torch.zeros(g.batch, dtype=torch.int32, device=device)
        ws = dion.api.workspace_for(g.m, g.n, g.batch, g.rank, device)
        idx = sorted(set([0, g.batch - 1][:sample]))
        for t in range(1, steps + 1):
            G = W.make_grad(wl, gi, t)
            Gd = to_torch(G, device)
            pre = {"X": to_numpy(Xd[idx]), "M": to_numpy(Md[idx]), "Q": to_numpy(Qd[idx])}
            Bpre = (Md.double() + Gd.double()) if g.rank == min(g.m, g.n) else None
            print(f"[fullsize] {wl.name} group {gi} step {t}: GPU step", flush=True)
            dion.step_(Xd, Gd, Md, Qd, g.rank, wl.mu, wl.lr, wl.eps, workspace=ws, flags=flags,
                       options=dion.OPT_STICKY_F64)
            torch.cuda.synchronize()
            P = ws[:4 * g.batch * g.m * g.rank].view(torch.float32).view(g.batch, g.m, g.rank)
            # properties on every matrix
            orth = 0.0
            for i in range(g.batch):
                Pi = P[i].double()
                orth = max(orth, float((Pi.T @ Pi - torch.eye(g.rank, dtype=torch.float64, device=device))
                                       .abs().max()))
            fr = None
            if Bpre is not None:
                fr = max(float(torch.linalg.norm(Md[i].double() - wl.mu * Bpre[i]) / torch.linalg.norm(Bpre[i]))
                         for i in range(g.batch))
            fl = to_numpy(flags)
            post = {"X": to_numpy(Xd[idx]), "M": to_numpy(Md[idx]), "Q": to_numpy(Qd[idx]), "P": to_numpy(P[idx])}
            print(f"[fullsize] {wl.name} group {gi} step {t}: oracle on matrices {idx}", flush=True)
            errs = compare_step(wl, pre, post, G[idx], g.rank)
            out.append(dict(group=gi, step=t, errs=errs, orth=orth, fullrank_M=fr, flags=fl))
            print(f"[fullsize]   orth={orth:.2e} fullrank_M={fr} flags={np.unique(fl).tolist()} "
                  f"errs={[{k: round(v, 9) for k, v in e.items() if k != 'rank_deficient'} for e in errs]}",
                  flush=True)
            del Gd, G
    return out


def _check(wl, res):
    tol = tol_for(wl)
    for r in res:
        assert not np.any(r["flags"] & 2), r
        assert r["orth"] <= 1e-4, r
        if r["fullrank_M"] is not None:
            assert r["fullrank_M"] <= tol, r
        for e in r["errs"]:
            for k in ("PQ", "M", "X"):
                assert e[k] <= tol, (r["group"], r["step"], k, e[k])


@pytest.mark.parametrize("wid,steps,sample", [(1, 3, 1), (2, 2, 2), (4, 1, 1)])
def test_full_size(cuda, wid, steps, sample):
    wl = W.get(wid)
    _check(wl, _run(wl, cuda, steps, sample))


def test_full_size_bf16_llama_stack(cuda):
    wl = W.get(3)
    _check(wl, _run(wl, cuda, 1, 1))


def test_full_size_full_rank(cuda):
    wl = W.get(5)
    _check(wl, _run(wl, cuda, 1, 1))
