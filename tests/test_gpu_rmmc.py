"""The relative maximum momentum change (RMMC) output of dion_step_batched_ex on the GPU.

  * against the oracle, teacher-forced (the oracle's M' from the GPU's pre-step state), to the
    workload's tolerance; against the same statistic taken on the host from the GPU's own M
    and M', to fp32 rounding (this pins the kernels' reduction itself);
  * closed forms of the step: full rank with G = 0 leaves M' = mu M (RMMC = 1 - mu); rank 0
    leaves M' = M + G (RMMC = max |G| / max |M|); a matrix whose factorization breaks down takes
    the rank-0 step; M = 0 gives +inf;
  * the large-tile weight pass with ragged edges (vector and element epilogues) and chunking
    (bitwise).
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import dion_step
from oracle.rmmc_oracle import rmmc as rmmc_oracle
from tests.harness import to_numpy, to_torch, tol_for

pytestmark = pytest.mark.gpu


def _host_rmmc(M_pre, M_post):
    return rmmc_oracle(M_pre.astype(np.float64), M_post.astype(np.float64))


def _step(wl, gi, device, X, M, Q, G, options=0, chunks=0):
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    from rank_orthonormalized_optimizer_amd._lib import opt_chunks
    g = wl.groups[gi]
    Xd, Md, Gd = to_torch(X, device), to_torch(M, device), to_torch(G, device)
    Qd = to_torch(Q, device) if g.rank else None
    out = torch.full((g.batch,), -1.0, dtype=torch.float32, device=device)
    flags = torch.zeros(g.batch, dtype=torch.int32, device=device)
    dion.step_(Xd, Gd, Md, Qd, g.rank, wl.mu, wl.lr, wl.eps, flags=flags, rmmc=out,
               options=options | (opt_chunks(chunks) if chunks else 0))
    torch.cuda.synchronize()
    return to_numpy(out), to_numpy(Md), to_numpy(flags)


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_rmmc_against_oracle(cuda, wid):
    wl = W.SMALL[wid]
    tol = tol_for(wl)
    for gi, g in enumerate(wl.groups):
        X, M, Q = W.make_state(wl, gi)
        # a non-zero momentum entering the step (step 1 from M = 0 would only test +inf)
        M[:] = W.store(1e-2 * np.random.default_rng(wid * 10 + gi).standard_normal(M.shape), "f32")
        G = W.make_grad(wl, gi, 1)
        print(f"[rmmc] {wl.name} group {gi} {g}", flush=True)
        got, Mn, _ = _step(wl, gi, cuda, X, M, Q, G)
        for i in range(g.batch):
            o = dion_step(W.to_f64(X[i], wl.x_dtype), W.to_f64(G[i], wl.g_dtype), M[i].astype(np.float64),
                          Q[i].astype(np.float64), wl.mu, wl.lr, wl.eps)
            ref = rmmc_oracle(M[i], o["M"])
            assert abs(got[i] - ref) <= tol * ref, (i, got[i], ref)
            own = _host_rmmc(M[i], Mn[i])
            assert abs(got[i] - own) <= 1e-6 * own, (i, got[i], own)


@pytest.mark.parametrize("shape", [(2, 64, 64), (3, 96, 80), (2, 80, 96)])
def test_rmmc_full_rank_without_gradient(cuda, shape):
    b, m, n = shape
    r = min(m, n)
    wl = W.SMALL[1].with_groups(W.Group(b, m, n, r), name="rmmc-full-rank")
    rng = np.random.default_rng(m * n)
    X = W.store(0.02 * rng.standard_normal((b, m, n)), "f32")
    M = W.store(1e-2 * rng.standard_normal((b, m, n)), "f32")
    Q = W.store(rng.standard_normal((b, n, r)) / math.sqrt(n), "f32")
    got, _, _ = _step(wl, 0, cuda, X, M, Q, np.zeros((b, m, n), np.float32))
    assert np.allclose(got, 1.0 - wl.mu, rtol=1e-4, atol=0), got


@pytest.mark.parametrize("gdt", ["f32", "bf16"])
def test_rmmc_rank0_and_zero_momentum(cuda, gdt):
    wl = (W.SMALL[1] if gdt == "f32" else W.SMALL[3]).with_groups(W.Group(3, 130, 200, 0), name="rmmc-rank0")
    rng = np.random.default_rng(7)
    X = W.store(0.02 * rng.standard_normal((3, 130, 200)), wl.x_dtype)
    M = W.store(1e-2 * rng.standard_normal((3, 130, 200)), "f32")
    M[2] = 0.0
    G = W.store(1e-3 * rng.standard_normal((3, 130, 200)), gdt)
    got, Mn, _ = _step(wl, 0, cuda, X, M, np.zeros((3, 200, 0), np.float32), G)
    for i in range(2):
        ref = np.abs(W.to_f64(G[i], gdt)).max() / np.abs(M[i]).max()
        assert abs(got[i] - ref) <= 1e-6 * ref, (i, got[i], ref)
        own = _host_rmmc(M[i], Mn[i])
        assert abs(got[i] - own) <= 1e-6 * own, (i, got[i], own)
    assert got[2] == np.inf


def test_rmmc_of_a_failed_matrix_is_the_rank0_one(cuda):
    import rank_orthonormalized_optimizer_amd as dion
    wl = W.SMALL[1].with_groups(W.Group(3, 256, 320, 24), name="rmmc-failed")
    X, M, Q = W.make_state(wl, 0)
    Q[1][:, 5] = 0.0
    M[:] = W.store(1e-2 * np.random.default_rng(3).standard_normal(M.shape), "f32")
    G = W.make_grad(wl, 0, 1)
    got, Mn, fl = _step(wl, 0, cuda, X, M, Q, G, options=dion.OPT_FORCE_F32)
    assert fl[1] & dion.FLAG_NONFINITE
    ref = np.abs(G[1].astype(np.float64)).max() / np.abs(M[1]).max()
    assert abs(got[1] - ref) <= 1e-6 * ref, (got[1], ref)


@pytest.mark.parametrize("base", [1, 3])
def test_rmmc_large_tiles_and_chunks(cuda, base):
    """16 x 520 x 1000 (both edges ragged, so the large-tile weight pass runs its vector and its
    element epilogues): against the host statistic of the GPU's own M, M'; chunks bitwise."""
    wl = W.SMALL[base].with_groups(W.Group(16, 520, 1000, 72), name=f"rmmc-wide-{base}")
    X, M, Q = W.make_state(wl, 0)
    M[:] = W.store(1e-2 * np.random.default_rng(base).standard_normal(M.shape), "f32")
    G = W.make_grad(wl, 0, 1)
    got, Mn, _ = _step(wl, 0, cuda, X, M, Q, G)
    for i in range(16):
        own = _host_rmmc(M[i], Mn[i])
        assert abs(got[i] - own) <= 1e-6 * own, (i, got[i], own)
    got3, Mn3, _ = _step(wl, 0, cuda, X, M, Q, G, chunks=3)
    assert np.array_equal(got.view(np.uint32), got3.view(np.uint32)) and np.array_equal(Mn, Mn3)
