"""GPU parity: the HIP step against the fp64 oracle, teacher-forced, per step.

Reduced-size versions of the five workloads (same recipes, shapes spanning
several 64-wide tiles with ragged tails) are compared element by element
through P Q^T, M and X, to 1e-4 relative Frobenius error for fp32 weights and
2e-2 for bf16 weights.
"""
import numpy as np
import pytest

import workloads as W
from tests.harness import TOL_KEYS, arith_for, check_errs, compare_step, to_numpy, to_torch, tol_for

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
            errs = compare_step(wl, pre, post, G, g.rank, arith=arith_for(wl, options))
            report.append((gi, t, errs, to_numpy(flags)))
    return report


def check(report, tol):
    worst = {}
    for gi, t, errs, flags in report:
        for i, e in enumerate(errs):
            where = f"group {gi} step {t} matrix {i}"
            assert not (flags[i] & 2), f"{where}: non-finite flag"
            for k in TOL_KEYS + ("Xband",):
                if k in e:
                    worst[k] = max(worst.get(k, 0.0), e[k])
            check_errs(e, tol, where)
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


@pytest.mark.parametrize("decades", [3.0, 5.0])
def test_near_identity_regimes(cuda, decades):
    """The fp64 second pass in each of its regimes, picked on the device by ||P^T P - I||_F after
    the first pass.  At step 1 (fp64 CholeskyQR of P0 on the host): with 3 decades of spectrum
    both matrices end below 1e-6 (first-order form); with 5 decades they end at 8e-5 and 2e-3
    (blocked Cholesky pass)."""
    import dataclasses
    import rank_orthonormalized_optimizer_amd as dion
    wl = dataclasses.replace(W.SMALL[5], grad_args={"decades": decades}, name=f"regimes-{decades:g}")
    # the regimes above, recomputed here so the test states what it covers
    X, M, Q = W.make_state(wl, 0)
    G = W.make_grad(wl, 0, 1)
    eps = []
    for i in range(wl.groups[0].batch):
        P0 = G[i].astype(np.float64) @ Q[i].astype(np.float64)
        L = np.linalg.cholesky(P0.T @ P0)
        P1 = np.linalg.solve(L, P0.T).T
        eps.append(np.linalg.norm(P1.T @ P1 - np.eye(P1.shape[1])))
    print("[regimes] eps after first pass", eps, flush=True)
    if decades == 3.0:
        assert max(eps) < 1e-6
    else:
        assert min(eps) > 1e-6
    rep = run_teacher_forced(wl, cuda, options=dion.OPT_FORCE_F64, steps=2)
    check(rep, tol_for(wl))


def test_sticky_hint_is_bitwise_neutral(cuda):
    """Skipping the fp32 chain once every flag is fp64 (StickyF64Hint) changes no bit."""
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    wl = W.SMALL[2]
    g = wl.groups[0]
    X, M, Q = W.make_state(wl, 0)
    runs = []
    for use_hint in (False, True):
        Xd, Md, Qd = to_torch(X, cuda), to_torch(M, cuda), to_torch(Q, cuda)
        flags = torch.zeros(g.batch, dtype=torch.int32, device=cuda)
        hint = dion.StickyF64Hint(flags) if use_hint else None
        stream = torch.cuda.current_stream(cuda)
        seq = []
        for t in range(1, 6):
            Gd = to_torch(W.make_grad(wl, 0, 1 + (t - 1) % 3), cuda)
            opts = dion.OPT_STICKY_F64 if hint is None else hint.options(dion.OPT_STICKY_F64)
            dion.step_(Xd, Gd, Md, Qd, g.rank, wl.mu, wl.lr, wl.eps, flags=flags, options=opts, stream=stream)
            if hint is not None:
                hint.after_step(stream)
            torch.cuda.synchronize()
            seq.append((to_numpy(Xd), to_numpy(Md), to_numpy(Qd), to_numpy(flags), opts))
        runs.append(seq)
        if hint is not None:
            assert hint.all_f64, "the hint never saw an all-fp64 stack"
    assert any(o[4] & dion.OPT_FORCE_F64 for o in runs[1]), "the hint never engaged"
    for a, b in zip(runs[0], runs[1]):
        for x, y in zip(a[:4], b[:4]):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("base,n", [(1, 1000), (3, 1000), (1, 998), (3, 996)])
def test_wide_update_tiles(cuda, base, n):
    """A stack large enough for the 128 x 64 weight-pass tiles (16 x 520 x n: both edges ragged,
    r = 72 padded to 96 in the split planes), fp32 and bf16 weights.  With n = 1000 the interior
    tiles take the vectorized epilogue and the edge tiles the element-wise one; n = 998 (rows
    not 16-byte aligned) sends every tile to the element-wise epilogue.  bf16 weights with n = 996
    (a multiple of 4, not of 8) take the one-part split product and the streaming back-projection."""
    wl = W.SMALL[base].with_groups(W.Group(16, 520, n, 72), name=f"wide-tiles-{base}-{n}", steps=2)
    check(run_teacher_forced(wl, cuda), tol_for(wl))


@pytest.mark.parametrize("m,n", [(256, 512), (256, 448), (256, 480), (300, 512)])
def test_split_product_launch_kinds(cuda, m, n):
    """fp32-chain product, r = 128: with whole 128 x 128 tiles and whole slabs (m = 256; K = n =
    512, 448 or 480, i.e. 16, 14 or 15 slabs, leaving 7, 5 and 6 slabs to the drain after the
    steady loop) the launch takes the branch-free staging loop; m = 300 (a ragged row tile)
    takes the general one."""
    wl = W.SMALL[1].with_groups(W.Group(4, m, n, 128), name=f"split-product-{m}x{n}", steps=2)
    check(run_teacher_forced(wl, cuda), tol_for(wl))


@pytest.mark.parametrize("batch,m,n,r", [(4, 1000, 300, 200), (2, 2048, 512, 256), (3, 640, 384, 128)])
def test_fp32_chain_gram_splits(cuda, batch, m, n, r):
    """fp32-chain Gram and apply on the split-bf16 kernel.  The Gram's K = m is cut into
    partials summed in split order: m = 1000, r = 200 gives three splits (334, 334, 332 rows)
    over ragged 128-tiles; m = 2048, r = 256 eight splits, and its apply has whole tiles (the
    branch-free staging loop, with the triangular K limit per column tile); m = 640, r = 128
    two splits.  Every matrix must stay on the fp32 chain."""
    import rank_orthonormalized_optimizer_amd as dion
    wl = W.SMALL[1].with_groups(W.Group(batch, m, n, r), name=f"gram6-{batch}x{m}x{n}-r{r}", steps=2)
    rep = run_teacher_forced(wl, cuda)
    for _, _, _, flags in rep:
        assert not np.any(flags & dion.FLAG_F64), flags
    check(rep, tol_for(wl))


@pytest.mark.parametrize("wid", [1, 2, 3, 5])
def test_householder_fallback(cuda, wid):
    """The fp64 chain's last-resort Householder QR (taken where every CholeskyQR pass broke down),
    requested for every matrix: each matrix must report it, and the step must match the oracle."""
    import rank_orthonormalized_optimizer_amd as dion
    wl = W.SMALL[wid]
    rep = run_teacher_forced(wl, cuda, options=dion.OPT_FORCE_F64 | dion.OPT_HOUSEHOLDER, steps=2)
    for _, _, _, flags in rep:
        assert np.all(flags & dion.FLAG_HOUSEHOLDER) and np.all(flags & dion.FLAG_F64), flags
        assert not np.any(flags & dion.FLAG_NONFINITE), flags
    check(rep, tol_for(wl))


@pytest.mark.parametrize("shape", [(2, 700, 640, 600), (1, 1100, 700, 590)])
def test_blocked_householder(cuda, shape):
    """Ranks above 512 take the blocked Householder QR (32-column panels in compact WY form, the
    panel updates and the formation of Q as fp64 matrix-core products): ragged last panels, a
    square-ish and a tall shape, requested for every matrix, against the oracle."""
    import rank_orthonormalized_optimizer_amd as dion
    b, m, n, r = shape
    wl = W.SMALL[2].with_groups(W.Group(b, m, n, r), name=f"hh-blocked-{m}x{n}-r{r}", steps=2)
    rep = run_teacher_forced(wl, cuda, options=dion.OPT_FORCE_F64 | dion.OPT_HOUSEHOLDER, steps=2)
    for _, _, _, flags in rep:
        assert np.all(flags & dion.FLAG_HOUSEHOLDER) and np.all(flags & dion.FLAG_F64), flags
        assert not np.any(flags & dion.FLAG_NONFINITE), flags
    check(rep, tol_for(wl))


@pytest.mark.parametrize("spectral", [False, True])
@pytest.mark.parametrize("force64", [False, True])
def test_shifted_first_pass(cuda, force64, spectral):
    """8 decades of spectrum: the fp64 chain's plain Cholesky of P0^T P0 breaks down (host fp64
    Cholesky fails too) and the shifted first pass plus two plain passes take over; shifted
    CholeskyQR3 in fp64 on the host stays within 4e-9 of the oracle's P Q^T on these inputs.
    With the spectral option the shift comes from the multi-power-iteration estimate of
    lambda_max(P0^T P0) instead of its trace; the passes must still succeed without the
    Householder last resort."""
    import dataclasses
    import rank_orthonormalized_optimizer_amd as dion
    wl = dataclasses.replace(W.SMALL[5], grad_args={"decades": 8.0}, name="shifted-8")
    opts = (dion.OPT_FORCE_F64 if force64 else 0) | (dion.OPT_SPECTRAL_SHIFT if spectral else 0)
    rep = run_teacher_forced(wl, cuda, options=opts, steps=2)
    for _, t, _, flags in rep:
        if t == 1:
            assert np.all(flags & dion.FLAG_SHIFTED), flags
        assert not np.any(flags & (dion.FLAG_HOUSEHOLDER | dion.FLAG_NONFINITE)), flags
    check(rep, tol_for(wl))


def test_spectral_shift_chunks_bitwise(cuda):
    """The spectral shift's pool lives in per-matrix workspace slices: splitting the stack into
    concurrent chunks must not change a bit of the shifted step."""
    import dataclasses
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    from rank_orthonormalized_optimizer_amd._lib import opt_chunks
    wl = dataclasses.replace(W.SMALL[5], grad_args={"decades": 8.0}, name="shifted-8-chunks")
    g = wl.groups[0]
    X, M, Q = W.make_state(wl, 0)
    G = to_torch(W.make_grad(wl, 0, 1), cuda)
    outs = []
    for nc in (1, 2):
        Xd, Md, Qd = to_torch(X, cuda), to_torch(M, cuda), to_torch(Q, cuda)
        flags = torch.zeros(g.batch, dtype=torch.int32, device=cuda)
        print(f"[parity] spectral shift chunks={nc}", flush=True)
        dion.step_(Xd, G, Md, Qd, g.rank, wl.mu, wl.lr, wl.eps, flags=flags,
                   options=dion.OPT_FORCE_F64 | dion.OPT_SPECTRAL_SHIFT | opt_chunks(nc))
        torch.cuda.synchronize()
        outs.append((to_numpy(Xd), to_numpy(Md), to_numpy(Qd), to_numpy(flags)))
    assert np.all(outs[0][3] & dion.FLAG_SHIFTED)
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("exact", [False, True])
def test_bf16_weight_arithmetic(cuda, exact):
    """bf16 weights: plain bf16 products by default (within the bf16 tolerance), the fp32-accurate
    split with OPT_EXACT_PRODUCTS (then P Q'^T and the momentum update match the oracle to fp32
    accuracy; X' differs from the oracle's unrounded X' by its bf16 rounding only)."""
    import rank_orthonormalized_optimizer_amd as dion
    wl = W.SMALL[3]
    rep = run_teacher_forced(wl, cuda, options=dion.OPT_EXACT_PRODUCTS if exact else 0)
    worst = check(rep, tol_for(wl))
    if exact:
        assert worst["PQ"] <= 1e-4 and worst["dM"] <= 1e-4 and worst["M"] <= 1e-4, worst
    else:
        assert worst["PQ"] > 1e-4, "plain bf16 products should show bf16-level error"
