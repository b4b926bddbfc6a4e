"""The GPU parity checks can fail: run them on an emulated step (CPU, numpy) whose
weight pass is done the way the kernels do it (fp32 P, R, Q' products, fp32 M', X'
rounded to the storage type), once correctly and once with each of several planted
mistakes in the update.  The correct emulation must pass every check; each mistake
must fail at least one."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import dion_step
from tests.harness import check_errs, compare_step, tol_for


def _rb(a):
    """RNE_bf16 of fp32 values, as fp32."""
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.asarray(a, np.float32)))


def _split2(a):
    """hi + lo of fp32 values: hi = RNE_bf16(a), lo = RNE_bf16(a - hi), as fp64."""
    a = np.asarray(a, np.float32)
    hi = _rb(a)
    return hi.astype(np.float64), _rb(a - hi).astype(np.float64)


def _prod3(a, b):
    """a b^T from two-part operands, the hi hi, hi lo and lo hi products only (then fp32)."""
    ah, al = _split2(a)
    bh, bl = _split2(b)
    return (ah @ bh.T + ah @ bl.T + al @ bh.T).astype(np.float32)


def _emulated_step(wl, gi, mistake=None, arith="split6"):
    g = wl.groups[gi]
    X, M, Q = W.make_state(wl, gi)
    G = W.make_grad(wl, gi, 1)
    post = {"X": X.copy(), "M": M.copy(), "Q": Q.copy(), "P": np.empty((g.batch, g.m, g.rank), np.float32)}
    lr_s = np.float32(wl.lr * math.sqrt(g.m / g.n))
    omm = np.float32(1.0 - wl.mu)
    if mistake == "scale":
        lr_s = np.float32(lr_s * 1.01)
    if mistake == "scale30":
        lr_s = np.float32(lr_s * 1.3)
    # the products' operands: fp32 (the exact split) or rounded once to bf16 (plain bf16)
    op = (lambda a: a) if arith == "split6" else _rb
    if mistake == "mu":
        omm = np.float32(omm * 1.01)
    for i in range(g.batch):
        o = dion_step(W.to_f64(X[i], wl.x_dtype), W.to_f64(G[i], wl.g_dtype), M[i].astype(np.float64),
                      Q[i].astype(np.float64), wl.mu, wl.lr, wl.eps)
        P32, R32, Q32 = o["P"].astype(np.float32), o["R"].astype(np.float32), o["Q"].astype(np.float32)
        B32 = M[i] + W.to_f64(G[i], wl.g_dtype).astype(np.float32)
        prod = _prod3 if arith == "split3" else (lambda a, b: op(a) @ op(b).T)
        upd_m = prod(P32, R32)
        if mistake == "no_feedback":
            upd_m = np.zeros_like(upd_m)
        post["M"][i] = B32 - omm * upd_m
        upd_x = prod(P32, Q32)
        if mistake == "q_rows_reversed":     # a wrong row index into Q'
            upd_x = prod(P32, Q32[::-1])
        x = W.to_f64(X[i], wl.x_dtype).astype(np.float32) - lr_s * upd_x
        if mistake == "no_update":
            x = W.to_f64(X[i], wl.x_dtype).astype(np.float32)
        post["X"][i] = W.f32_to_bf16_bits(x) if wl.x_dtype == "bf16" else x
        post["Q"][i] = Q32
        post["P"][i] = P32
    return compare_step(wl, {"X": X, "M": M, "Q": Q}, post, G, g.rank, arith=arith)


def _fails(errs, tol):
    try:
        for e in errs:
            check_errs(e, tol)
    except AssertionError:
        return True
    return False


# fp32 weights: SMALL[1] (256 x 512, r = 32); bf16 weights: the first stack of SMALL[3]
CASES = {"f32": W.SMALL[1], "bf16": W.SMALL[3]}


@pytest.mark.parametrize("case,arith", [("f32", "split6"), ("f32", "split3"), ("bf16", "split6"), ("bf16", "bf16")])
def test_correct_emulation_passes(case, arith):
    wl = CASES[case]
    errs = _emulated_step(wl, 0, arith=arith)
    for e in errs:
        check_errs(e, tol_for(wl))
        assert e["Xband"] == 0


@pytest.mark.parametrize("case,mistake", [
    ("f32", "no_update"), ("f32", "scale"), ("f32", "mu"), ("f32", "no_feedback"), ("f32", "q_rows_reversed"),
    ("bf16", "no_update"), ("bf16", "scale"), ("bf16", "q_rows_reversed"), ("bf16", "no_feedback"),
])
def test_planted_update_mistake_is_caught(case, mistake):
    wl = CASES[case]
    assert _fails(_emulated_step(wl, 0, mistake), tol_for(wl)), mistake


@pytest.mark.parametrize("mistake", ["no_update", "scale", "mu", "q_rows_reversed", "no_feedback"])
def test_planted_mistake_is_caught_with_two_part_products(mistake):
    """The two-part split of fp32 weights widens the band to about 3 * 2^-16 of |P| |Q'|^T."""
    wl = CASES["f32"]
    assert _fails(_emulated_step(wl, 0, mistake, arith="split3"), tol_for(wl)), mistake


@pytest.mark.parametrize("mistake", ["no_update", "scale30", "q_rows_reversed", "no_feedback"])
def test_planted_mistake_is_caught_with_plain_bf16_products(mistake):
    """Plain bf16 products widen the element-wise band to the bf16 rounding of the operands
    (about 2^-7 of |P| |Q'|^T); mistakes beyond the bf16 tolerance are still caught."""
    wl = CASES["bf16"]
    assert _fails(_emulated_step(wl, 0, mistake, arith="bf16"), tol_for(wl)), mistake
