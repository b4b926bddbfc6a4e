"""Degenerate cases of the method, on the GPU, through the C ABI.

  rank 0          the update is zero: M' = M + G (fp32 add, bitwise), X untouched, Q may be NULL;
  no factor       a factorization that breaks down with no fallback left (DION_OPT_FORCE_F32 and a
                  zero column of Q, so the first Cholesky pivot of that column is exactly 0): that
                  matrix takes the rank-0 step (M' = M + G, X and Q bitwise untouched) and is
                  flagged non-finite, while the rest of the stack steps normally;
  natural breakdown  Q with a duplicated column or a zero column makes P0 = B Q singular, so every
                  CholeskyQR pass breaks down and the fp64 Householder QR takes the matrix without
                  being asked to (no DION_OPT_HOUSEHOLDER).  The Q-factor is then not unique past the
                  degenerate column: checked are P^T P = I, the identity B = M' + (1 - mu) P R^T
                  with R = B^T P, the leading columns of P (unique) against the oracle, and the
                  weight pass element by element; the other matrices of the stack against the
                  oracle in full.
"""
import numpy as np
import pytest

import workloads as W
from oracle import dion_step
from tests.harness import check_errs, compare_step, rel, to_numpy, to_torch, tol_for

pytestmark = pytest.mark.gpu


def _f32_add(M, G, g_dtype):
    return (M + W.to_f64(G, g_dtype).astype(np.float32)).astype(np.float32)


@pytest.mark.parametrize("xdt,gdt", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
@pytest.mark.parametrize("shape", [(3, 200, 136), (1, 1, 1), (2, 64, 1000)])
def test_rank0_through_abi(cuda, xdt, gdt, shape):
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    from rank_orthonormalized_optimizer_amd import _lib
    b, m, n = shape
    rng = np.random.default_rng(b * 1000 + m + n)
    X = W.store(0.02 * rng.standard_normal((b, m, n)), xdt)
    G = W.store(1e-2 * rng.standard_normal((b, m, n)), gdt)
    M = (1e-2 * rng.standard_normal((b, m, n))).astype(np.float32)
    Xd, Gd, Md = to_torch(X, cuda), to_torch(G, cuda), to_torch(M, cuda)
    flags = torch.full((b,), 7, dtype=torch.int32, device=cuda)
    nbytes = _lib.workspace_size(m, n, b, 0)
    ws = dion.api.workspace_for(m, n, b, 0, cuda)
    dt = {"f32": _lib.F32, "bf16": _lib.BF16}
    print(f"[edge] rank 0 {shape} X {xdt} G {gdt}", flush=True)
    st = _lib.step_batched_raw(Xd.data_ptr(), Gd.data_ptr(), Md.data_ptr(), 0, m, n, b, 0, 0.95, 0.01, 1e-8,
                               dt[xdt], dt[gdt], ws.data_ptr(), nbytes, flags.data_ptr(), 0,
                               int(torch.cuda.current_stream(cuda).cuda_stream))
    assert st == _lib.OK, _lib.strerror(st)
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(Md).view(np.uint32), _f32_add(M, G, gdt).view(np.uint32))
    assert np.array_equal(to_numpy(Xd), X)
    assert np.array_equal(to_numpy(flags), np.zeros(b, np.int32))


def _zero_column_case():
    wl = W.SMALL[1].with_groups(W.Group(3, 256, 320, 24), name="zero-column", steps=1)
    X, M, Q = W.make_state(wl, 0)
    Q[1][:, 5] = 0.0
    return wl, X, M, Q


def test_failed_factorization_takes_the_rank0_step(cuda):
    """FORCE_F32 and a zero column of Q in matrix 1: its fp32 Cholesky pivot is exactly 0 and
    there is no fallback, so it gets M' = M + G and keeps X and Q; matrices 0 and 2 step normally."""
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    wl, X, M, Q = _zero_column_case()
    g = wl.groups[0]
    G = W.make_grad(wl, 0, 1)
    # a non-zero momentum, so that M' = M + G is not just G
    M[:] = W.store(1e-2 * np.random.default_rng(3).standard_normal(M.shape), "f32")
    Xd, Gd, Md, Qd = to_torch(X, cuda), to_torch(G, cuda), to_torch(M, cuda), to_torch(Q, cuda)
    flags = torch.zeros(g.batch, dtype=torch.int32, device=cuda)
    ws = dion.api.workspace_for(g.m, g.n, g.batch, g.rank, cuda)
    print("[edge] failed factorization under FORCE_F32", flush=True)
    dion.step_(Xd, Gd, Md, Qd, g.rank, wl.mu, wl.lr, wl.eps, workspace=ws, flags=flags,
               options=dion.OPT_FORCE_F32)
    torch.cuda.synchronize()
    fl = to_numpy(flags)
    assert fl[1] & dion.FLAG_NONFINITE and not (fl[1] & dion.FLAG_F64), fl
    assert not (fl[0] & dion.FLAG_NONFINITE) and not (fl[2] & dion.FLAG_NONFINITE), fl
    Mn, Xn, Qn = to_numpy(Md), to_numpy(Xd), to_numpy(Qd)
    assert np.array_equal(Mn[1].view(np.uint32), _f32_add(M[1], G[1], "f32").view(np.uint32))
    assert np.array_equal(Xn[1], X[1]) and np.array_equal(Qn[1], Q[1])
    P = ws[:4 * g.batch * g.m * g.rank].view(torch.float32).view(g.batch, g.m, g.rank)
    post = {"X": Xn, "M": Mn, "Q": Qn, "P": to_numpy(P)}
    for e, i in zip(compare_step(wl, {"X": X, "M": M, "Q": Q}, post, G, g.rank, idx=[0, 2]), (0, 2)):
        check_errs(e, tol_for(wl), f"matrix {i}")


@pytest.mark.parametrize("kind,shape", [("duplicate", (3, 256, 320, 24)), ("zero", (3, 256, 320, 24)),
                                        ("duplicate", (2, 640, 600, 560))])
def test_natural_breakdown_reaches_householder(cuda, kind, shape):
    """A degenerate Q column makes P0 singular: every CholeskyQR pass breaks down and the matrix
    reaches the Householder QR without the option (the blocked form at rank 560)."""
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    wl = W.SMALL[1].with_groups(W.Group(*shape), name=f"breakdown-{kind}-r{shape[3]}", steps=2)
    g = wl.groups[0]
    X, M, Q = W.make_state(wl, 0)
    j = 7
    if kind == "duplicate":
        Q[1][:, j] = Q[1][:, 2]
    else:
        Q[1][:, j] = 0.0
    Xd, Md, Qd = to_torch(X, cuda), to_torch(M, cuda), to_torch(Q, cuda)
    flags = torch.zeros(g.batch, dtype=torch.int32, device=cuda)
    ws = dion.api.workspace_for(g.m, g.n, g.batch, g.rank, cuda)
    for t in (1, 2):
        G = W.make_grad(wl, 0, t)
        pre = {"X": to_numpy(Xd), "M": to_numpy(Md), "Q": to_numpy(Qd)}
        print(f"[edge] natural breakdown ({kind} column) step {t}", flush=True)
        dion.step_(Xd, to_torch(G, cuda), Md, Qd, g.rank, wl.mu, wl.lr, wl.eps, workspace=ws, flags=flags,
                   options=dion.OPT_STICKY_F64)
        torch.cuda.synchronize()
        fl = to_numpy(flags)
        P = to_numpy(ws[:4 * g.batch * g.m * g.rank].view(torch.float32).view(g.batch, g.m, g.rank))
        post = {"X": to_numpy(Xd), "M": to_numpy(Md), "Q": to_numpy(Qd), "P": P}
        errs = compare_step(wl, pre, post, G, g.rank)
        print(f"[edge]   flags {fl.tolist()} errs {errs}", flush=True)
        assert not np.any(fl & dion.FLAG_NONFINITE), fl
        if t == 1:   # step 1 starts from the degenerate Q; after it Q' = colnorm(B^T P) is regular
            assert fl[1] & dion.FLAG_HOUSEHOLDER and fl[1] & dion.FLAG_F64, fl
            assert errs[1]["rank_deficient"]
        for i, e in enumerate(errs):
            assert e["orth"] <= 1e-4, (i, e)
            assert e["Xband"] == 0, (i, e)
            if e["rank_deficient"]:
                Bm = pre["M"][i].astype(np.float64) + G[i].astype(np.float64)
                Pi = P[i].astype(np.float64)
                Mi = post["M"][i].astype(np.float64)
                assert rel(Mi + (1 - wl.mu) * Pi @ (Bm.T @ Pi).T, Bm) <= 1e-6
                # the Q-factor's columns before the degenerate one are unique
                o = dion_step(W.to_f64(pre["X"][i], "f32"), G[i].astype(np.float64), pre["M"][i].astype(np.float64),
                              pre["Q"][i].astype(np.float64), wl.mu, wl.lr, wl.eps)
                assert rel(Pi[:, :j], o["P"][:, :j]) <= 1e-4
            else:
                check_errs(e, tol_for(wl), f"step {t} matrix {i}")
