"""Pins of the fp64 oracle against what the pages and the mathematics fix.

The pages print no worked example of a Dion step, so nothing here is a stored
page number.  Instead every step is pinned by something other than itself:

  S1 B = M + G          exact rational sum (fractions.Fraction)
  S2 P0 = B Q           pure-Python triple loop with correctly rounded sums
  S3 P = orth(P0)       P^T P = I; P T = P0 with T upper triangular, diag > 0;
                        50-digit modified Gram-Schmidt (oracle/mp_reference.py)
  S4-S5 R, Q'           unit columns parallel to R at eps = 0; the eps form;
                        invariance of P Q'^T under B -> cB and column sign flips
  S6 M'                 projections P^T M' = mu P^T B and (I - P P^T) M' = (I - P P^T) B;
                        full rank: M' = mu B exactly
  S7 X'                 ||X - X'||_F = lr sqrt(m/n) sqrt(sum ||q_j||^2), = lr sqrt(m/n) sqrt(r) at eps = 0
  whole step            repeated steps on a fixed B converge to U_r V_r^T of a brute-force SVD,
                        and at full rank to msgn(B) = U V^T (the DeMuon page's
                        "Ortogonalización de Matrices"); rank 0 leaves X unchanged and M = M + G
  fixtures              tests/golden/tiny_steps_mp50.json (50-digit step, different QR algorithm)

The mutation tests at the end plant plausible mistakes in the oracle (on the
CPU, by patching one of its step functions) and check that a pin catches each.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.dion_oracle as O
import workloads as W
from oracle.mp_reference import dion_step_mp, mgs_qr

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_steps_mp50.json")


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def haar(rng, n):
    q, t = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(t))


def wl_inputs(wid, step=1, gi=0):
    wl = W.SMALL[wid]
    X, M, Q = W.make_state(wl, gi)
    G = W.make_grad(wl, gi, step)
    return wl, W.to_f64(X[0], wl.x_dtype), W.to_f64(G[0], wl.g_dtype), M[0].astype(np.float64), Q[0].astype(
        np.float64)


# ----------------------------------------------------------------------------- pins
def pin_accumulate_exact():
    rng = np.random.default_rng(1)
    M = (rng.standard_normal(400) * 10.0 ** rng.uniform(-6, 3, 400)).astype(np.float32)
    G32 = (rng.standard_normal(400) * 10.0 ** rng.uniform(-6, 3, 400)).astype(np.float32)
    Gbf = W.bf16_bits_to_f32(W.f32_to_bf16_bits(G32))
    for G in (G32, Gbf):
        B = O.accumulate(M.astype(np.float64), G.astype(np.float64))
        for i in range(400):
            exact = Fraction(float(M[i])) + Fraction(float(G[i]))
            # fp64 addition is correctly rounded; it is exact when the fp32 exponents differ by <= 29
            assert float(B[i]) == float(exact), i
            if M[i] != 0 and G[i] != 0 and abs(math.frexp(float(M[i]))[1] - math.frexp(float(G[i]))[1]) <= 29:
                assert Fraction(float(B[i])) == exact, i


def pin_power_step_bruteforce():
    rng = np.random.default_rng(2)
    B = rng.standard_normal((7, 9))
    Q = rng.standard_normal((9, 4))
    P0 = O.power_step(B, Q)
    for i in range(7):
        for j in range(4):
            exact = math.fsum(float(B[i, k]) * float(Q[k, j]) for k in range(9))
            assert abs(P0[i, j] - exact) <= 1e-15 * max(1.0, abs(exact)) * 9


def pin_qr_properties():
    for wid in (1, 2, 4, 5):
        wl, X, G, M, Q = wl_inputs(wid)
        P0 = O.power_step(O.accumulate(M, G), Q)
        P, T = O.thin_qr_positive(P0)
        r = Q.shape[1]
        assert np.abs(P.T @ P - np.eye(r)).max() <= 1e-10, wid
        assert np.allclose(np.tril(T, -1), 0.0), wid
        assert np.all(np.diag(T) > 0), wid
        assert rel(P @ T, P0) <= 1e-12, wid


def pin_qr_vs_mp50():
    rng = np.random.default_rng(3)
    for (m, r) in ((6, 4), (9, 3), (5, 5)):
        P0 = rng.standard_normal((m, r))
        P, T = O.thin_qr_positive(P0)
        import mpmath as mp
        with mp.workdps(50):
            Pm, Tm = mgs_qr([[mp.mpf(float(v)) for v in row] for row in P0])
            Pm = np.array([[float(v) for v in row] for row in Pm])
            Tm = np.array([[float(v) for v in row] for row in Tm])
        assert np.abs(P - Pm).max() <= 1e-14, (m, r)
        assert np.abs(T - Tm).max() <= 1e-13 * np.abs(Tm).max(), (m, r)


def pin_golden_mp50():
    d = json.load(open(GOLDEN))
    for case in d["cases"]:
        c, inp, exp = case["case"], case["inputs"], case["expected"]
        o = O.dion_step(np.array(inp["X"]), np.array(inp["G"]), np.array(inp["M"]), np.array(inp["Q"]),
                        c["mu"], c["lr"], c["eps"])
        for k in ("X", "M", "Q", "P"):
            assert rel(o[k], np.array(exp[k])) <= 1e-13, (c["name"], k, rel(o[k], np.array(exp[k])))
        assert rel(o["P"] @ o["Q"].T, np.array(exp["PQ"])) <= 1e-13, c["name"]


def pin_colnorm():
    wl, X, G, M, Q = wl_inputs(4)
    o = O.dion_step(X, G, M, Q, wl.mu, wl.lr, 0.0)
    Qn, R = o["Q"], o["R"]
    assert np.abs(np.linalg.norm(Qn, axis=0) - 1.0).max() <= 1e-13
    cos = np.sum(Qn * R, axis=0) / (np.linalg.norm(Qn, axis=0) * np.linalg.norm(R, axis=0))
    assert np.abs(cos - 1.0).max() <= 1e-13
    # eps enters as ||r_j|| + eps: q_j (||r_j|| + eps) = r_j
    eps = 0.3 * float(np.median(np.linalg.norm(R, axis=0)))
    o2 = O.dion_step(X, G, M, Q, wl.mu, wl.lr, eps)
    nr = np.sqrt(np.array([math.fsum(float(v) ** 2 for v in R[:, j]) for j in range(R.shape[1])]))
    assert rel(o2["Q"] * (nr + eps)[None, :], R) <= 1e-13


def pin_invariances():
    wl, X, G, M, Q = wl_inputs(1)
    base = O.dion_step(X, G, M, Q, wl.mu, wl.lr, 0.0)
    pq = base["P"] @ base["Q"].T
    scaled = O.dion_step(X, 3.7 * G, 3.7 * M, Q, wl.mu, wl.lr, 0.0)
    assert rel(scaled["P"] @ scaled["Q"].T, pq) <= 1e-12
    D = np.where(np.arange(Q.shape[1]) % 3 == 0, -1.0, 1.0)
    flipped = O.dion_step(X, G, M, Q * D[None, :], wl.mu, wl.lr, 0.0)
    assert rel(flipped["P"] @ flipped["Q"].T, pq) <= 1e-12
    assert rel(flipped["M"], base["M"]) <= 1e-12
    assert rel(flipped["X"], base["X"]) <= 1e-14


def pin_error_feedback_projections():
    for wid in (1, 2, 4):
        wl, X, G, M, Q = wl_inputs(wid)
        o = O.dion_step(X, G, M, Q, wl.mu, wl.lr, wl.eps)
        P, B, Mn = o["P"], o["B"], o["M"]
        nb = np.linalg.norm(B)
        assert np.linalg.norm(P.T @ Mn - wl.mu * (P.T @ B)) <= 1e-12 * nb, wid
        out_m = Mn - P @ (P.T @ Mn)
        out_b = B - P @ (P.T @ B)
        assert np.linalg.norm(out_m - out_b) <= 1e-12 * nb, wid


def pin_full_rank_momentum():
    rng = np.random.default_rng(4)
    for (m, n, mu) in ((40, 40, 0.9), (24, 50, 0.95), (50, 24, 0.5)):
        r = min(m, n)
        B = rng.standard_normal((m, n))
        Q = rng.standard_normal((n, r))
        o = O.dion_step(np.zeros((m, n)), B, np.zeros((m, n)), Q, mu, 0.01, 1e-8)
        assert rel(o["M"], mu * B) <= 1e-13, (m, n)


def pin_update_norm():
    for wid in (1, 4):
        wl, X, G, M, Q = wl_inputs(wid)
        m, n = X.shape
        r = Q.shape[1]
        o = O.dion_step(X, G, M, Q, wl.mu, wl.lr, 0.0)
        d = np.linalg.norm(X - o["X"])
        assert abs(d - wl.lr * math.sqrt(m / n) * math.sqrt(r)) <= 1e-9 * d, wid
        o2 = O.dion_step(X, G, M, Q, wl.mu, wl.lr, 1e-3)
        want = wl.lr * math.sqrt(m / n) * math.sqrt(float(np.sum(np.linalg.norm(o2["Q"], axis=0) ** 2)))
        assert abs(np.linalg.norm(X - o2["X"]) - want) <= 1e-9 * want, wid


def pin_power_iteration_limit():
    rng = np.random.default_rng(5)
    m, n = 14, 10
    U = haar(rng, m)[:, :n]
    V = haar(rng, n)
    sig = 2.0 ** (-np.arange(n))
    B = (U * sig[None, :]) @ V.T
    for r in (3, n):
        Q = rng.standard_normal((n, r))
        for _ in range(40):
            o = O.dion_step(np.zeros((m, n)), B, np.zeros((m, n)), Q, 0.9, 0.01, 0.0)
            Q = o["Q"]
        target = U[:, :r] @ V[:, :r].T
        assert rel(o["P"] @ o["Q"].T, target) <= 1e-10, r
    # full rank: the limit is the matrix sign msgn(B) = U V^T
    Us, _, Vt = np.linalg.svd(B, full_matrices=False)
    assert rel(o["P"] @ o["Q"].T, Us @ Vt) <= 1e-10


def pin_rank_zero():
    wl, X, G, M, Q = wl_inputs(1)
    M = M + 0.25
    o = O.dion_step(X, G, M, Q[:, :0], wl.mu, wl.lr, wl.eps)
    assert np.array_equal(o["X"], X)
    assert np.array_equal(o["M"], M + G)
    assert o["Q"].shape == (X.shape[1], 0)


def pin_batched():
    wl = W.SMALL[2]
    X, M, Q = W.make_state(wl, 0)
    G = W.make_grad(wl, 0, 1)
    ob = O.dion_step_batched(X.astype(np.float64), G.astype(np.float64), M.astype(np.float64),
                             Q.astype(np.float64), wl.mu, wl.lr, wl.eps)
    for i in range(X.shape[0]):
        oi = O.dion_step(X[i].astype(np.float64), G[i].astype(np.float64), M[i].astype(np.float64),
                         Q[i].astype(np.float64), wl.mu, wl.lr, wl.eps)
        for k in ("X", "M", "Q", "P"):
            assert np.array_equal(ob[k][i], oi[k])


PINS = [pin_accumulate_exact, pin_power_step_bruteforce, pin_qr_properties, pin_qr_vs_mp50, pin_golden_mp50,
        pin_colnorm, pin_invariances, pin_error_feedback_projections, pin_full_rank_momentum, pin_update_norm,
        pin_power_iteration_limit, pin_rank_zero, pin_batched]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_mp_reference_self_consistent():
    """The 50-digit step itself: orthonormal P, full-rank closed form M' = mu B."""
    rng = np.random.default_rng(6)
    m, n = 5, 4
    B = rng.standard_normal((m, n))
    Q = rng.standard_normal((n, n))
    o = dion_step_mp(np.zeros((m, n)), B, np.zeros((m, n)), Q, 0.9, 0.01, 1e-8)
    assert np.abs(o["P"].T @ o["P"] - np.eye(n)).max() <= 1e-15
    assert rel(o["M"], 0.9 * B) <= 1e-15


# ----------------------------------------------------------------------------- planted mistakes
def _qr_raw(P0):
    return np.linalg.qr(P0, mode="reduced")


def _qr_polar(P0):
    U, _, Vt = np.linalg.svd(P0, full_matrices=False)
    P = U @ Vt
    return P, P.T @ P0


MUTATIONS = {
    "accumulate_rounded_fp32": ("accumulate", lambda M, G: (M.astype(np.float32) + G.astype(np.float32))
                                .astype(np.float64)),
    "power_step_transposed_Q": ("power_step", lambda B, Q: B @ (Q[::-1])),
    "qr_without_sign_fix": ("thin_qr_positive", _qr_raw),
    "qr_polar_instead_of_qr": ("thin_qr_positive", _qr_polar),
    "project_back_uses_P0_scale": ("project_back", lambda B, P: 2.0 * (B.T @ P)),
    "feedback_sign_flipped": ("error_feedback", lambda B, P, R, mu: B + (1.0 - mu) * (P @ R.T)),
    "feedback_mu_swapped": ("error_feedback", lambda B, P, R, mu: B - mu * (P @ R.T)),
    "colnorm_by_rows": ("column_normalize",
                        lambda R, eps: R / (np.linalg.norm(R, axis=1, keepdims=True) + eps)),
    "colnorm_eps_as_max": ("column_normalize",
                           lambda R, eps: R / np.maximum(np.linalg.norm(R, axis=0, keepdims=True), eps)),
    "scale_inverted": ("update_scale", lambda m, n: math.sqrt(n / m)),
    "update_sign_flipped": ("weight_update", lambda X, P, Qn, lr, s: X + lr * s * (P @ Qn.T)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, np.linalg.LinAlgError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
