"""Pins of the multi-power-iteration oracle (oracle/spectral_oracle.py).

The DASH summary (gist.science, "Methodologie", the item on multi-power-iteration
scaling) describes the estimator without a worked example, so the pins are what
the mathematics fixes:

  bound        a Rayleigh quotient never exceeds lambda_max (LAPACK eigvalsh) nor falls
               below lambda_min
  rank one     W = a a^T: one product maps any start vector onto a, so the estimate is
               ||a||^2 exactly
  eigenvectors a pool of scaled eigenvectors of a diagonal W returns the largest of their
               eigenvalues exactly, for any iteration count (the pool's maximum, not its first
               vector, and the quotient divides by v^T v)
  rate         a start vector c1 u1 + c2 u2 gives the closed form
               (c1^2 l1^(2t+1) + c2^2 l2^(2t+1)) / (c1^2 l1^(2t) + c2^2 l2^(2t))
  convergence  a gapped spectrum reaches eigvalsh's lambda_max to 1e-12
  zero         W = 0 gives 0

The planted-mistake tests patch a mistake into a copy of the oracle (on the CPU) and
check that a pin fails for each.
"""
import numpy as np
import pytest

import oracle.spectral_oracle as S


def _psd(r, seed, decay=None):
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((r, r)))
    lam = rng.uniform(0.1, 1.0, r) if decay is None else decay ** np.arange(r)
    return (U * lam) @ U.T, U, lam


def pin_bound(est=S.lambda_max_estimate):
    for seed, r, k in ((1, 40, 8), (2, 17, 32), (3, 64, 3)):
        rng = np.random.default_rng(seed)
        A = rng.standard_normal((r, r + 5))
        W = A @ A.T
        ev = np.linalg.eigvalsh(W)
        for t in (0, 1, 3, 10):
            lam = est(W, rng.standard_normal((r, k)), t)
            assert ev[0] * (1 - 1e-12) <= lam <= ev[-1] * (1 + 1e-12), (seed, t)


def pin_rank_one(est=S.lambda_max_estimate):
    rng = np.random.default_rng(4)
    a = rng.standard_normal(33)
    W = np.outer(a, a)
    for t in (1, 2, 5):
        assert abs(est(W, rng.standard_normal((33, 4)), t) - a @ a) <= 1e-12 * (a @ a), t


def pin_eigenvectors(est=S.lambda_max_estimate):
    d = np.array([0.5, 3.0, 1.0, 7.0, 2.0, 0.25])
    W = np.diag(d)
    for cols, want in (([0, 1, 2], 3.0), ([2, 3, 5], 7.0), ([4], 2.0), ([5, 0], 0.5)):
        V0 = np.zeros((6, len(cols)))
        for j, c in enumerate(cols):
            V0[c, j] = 3.0 + j          # scaled: the quotient must divide by v^T v
        for t in (0, 1, 4):
            assert est(W, V0, t) == pytest.approx(want, rel=1e-15, abs=0), (cols, t)


def pin_rate(est=S.lambda_max_estimate):
    W, U, lam = _psd(12, 5)
    order = np.argsort(lam)[::-1]
    u1, u2 = U[:, order[0]], U[:, order[1]]
    l1, l2 = lam[order[0]], lam[order[1]]
    c1, c2 = 0.3, 2.0
    for t in range(0, 8):
        want = (c1 ** 2 * l1 ** (2 * t + 1) + c2 ** 2 * l2 ** (2 * t + 1)) / (c1 ** 2 * l1 ** (2 * t) + c2 ** 2 * l2 ** (2 * t))
        got = est(W, (c1 * u1 + c2 * u2)[:, None], t)
        assert got == pytest.approx(want, rel=1e-12), t


def pin_convergence(est=S.lambda_max_estimate):
    W, _, lam = _psd(48, 6, decay=0.7)
    rng = np.random.default_rng(7)
    got = est(W, rng.standard_normal((48, 32)), 60)
    assert got == pytest.approx(np.linalg.eigvalsh(W)[-1], rel=1e-12)


def pin_zero(est=S.lambda_max_estimate):
    assert est(np.zeros((5, 5)), np.ones((5, 2)), 3) == 0.0


PINS = [pin_bound, pin_rank_one, pin_eigenvectors, pin_rate, pin_convergence, pin_zero]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_batched_matches_single():
    rng = np.random.default_rng(8)
    W = np.stack([_psd(9, s)[0] for s in range(3)])
    V0 = rng.standard_normal((3, 9, 5))
    got = S.lambda_max_batched(W, V0, 4)
    assert [float(x) for x in got] == [S.lambda_max_estimate(W[i], V0[i], 4) for i in range(3)]


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        S.lambda_max_estimate(np.eye(3), np.ones((3, 1)), -1)
    with pytest.raises(ValueError):
        S.lambda_max_estimate(np.eye(3), np.ones((4, 1)), 1)


# planted mistakes: each must fail at least one pin
def _min_over_pool(W, V0, iters):
    return float(S.rayleigh_quotients(W, S.power_iterate(W, V0, iters)).min())


def _first_vector_only(W, V0, iters):
    return float(S.rayleigh_quotients(W, S.power_iterate(W, V0, iters))[0])


def _no_division_by_norm(W, V0, iters):
    V = S.power_iterate(W, V0, iters)
    return float(np.einsum("ij,ij->j", V, np.asarray(W) @ V).max())


def _one_iteration_short(W, V0, iters):
    return S.lambda_max_estimate(W, V0, max(iters - 1, 0))


def _norm_instead_of_quotient(W, V0, iters):   # ||W v|| / ||v||: the same at convergence, not before
    V = S.power_iterate(W, V0, iters)
    return float((np.linalg.norm(np.asarray(W) @ V, axis=0) / np.linalg.norm(V, axis=0)).max())


@pytest.mark.parametrize("bad,pins", [
    (_min_over_pool, [pin_eigenvectors]),
    (_first_vector_only, [pin_eigenvectors]),
    (_no_division_by_norm, [pin_eigenvectors]),
    (_one_iteration_short, [pin_rate]),
    (_norm_instead_of_quotient, [pin_rate, pin_bound]),
])
def test_planted_mistake_is_caught(bad, pins):
    caught = 0
    for pin in pins:
        try:
            pin(bad)
        except AssertionError:
            caught += 1
    assert caught > 0, f"{bad.__name__} passed every pin"


def test_start_vector_stream():
    """The counter-based start vectors: SplitMix64 seeded with 0 begins 0xe220a8397b1dcdaf,
    0x6e789e6aa1b965f4, 0x06c45d188009454f (its published reference outputs), and the vectors
    are 2u - 1 of the top 53 bits, row-major over (matrix, row, vector)."""
    import workloads as W
    z = W.splitmix64(np.array([1, 2, 3], dtype=np.uint64))
    assert [int(x) for x in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    v = W.splitmix_start_vectors(2, 3, 4)
    assert v[0, 0, 0] == 2.0 * (0xE220A8397B1DCDAF >> 11) / 2.0 ** 53 - 1.0
    assert v[1, 2, 3] == 2.0 * (int(W.splitmix64(np.array([24], dtype=np.uint64))[0]) >> 11) / 2.0 ** 53 - 1.0
    assert np.all(np.abs(v) < 1.0)
