"""Pins of the RMMC oracle against closed forms and the Dion step's own closed forms.

RMMC = max |M' - M| / max |M| per matrix (the reading of the CurvaDion abstract's
Relative Maximum Momentum Change).  Each pin is fixed by the definition or by the
mathematics of the step, not by retyping the formula:

  * no change gives 0; a single changed entry gives its change over the largest |M|,
    wherever the largest entries and the change sit and whatever their signs;
  * scaling M and M' by the same c != 0 leaves the value unchanged;
  * M = 0: 0 when M' = 0 as well, +inf otherwise;
  * the oracle's full-rank Dion step with G = 0 leaves M' = mu M exactly (P P^T B = B),
    so RMMC = 1 - mu; its rank-0 step leaves M' = M + G, so RMMC = max |G| / max |M|.

The planted mistakes (the new momentum as the scale, an element-wise relative change,
Frobenius norms in place of maxima) each fail a pin.
"""
import numpy as np
import pytest

from oracle import dion_step
from oracle.rmmc_oracle import rmmc


def pin_no_change(f=rmmc):
    M = np.random.default_rng(1).standard_normal((5, 7))
    assert f(M, M.copy()) == 0.0


def pin_single_entry(f=rmmc):
    M = np.array([[-4.0, 1.0, 0.5], [2.0, 3.0, -0.25]])
    for (i, j), d in (((0, 0), 0.5), ((1, 2), -1.0), ((0, 2), 2.0)):
        Mn = M.copy()
        Mn[i, j] += d
        assert f(M, Mn) == pytest.approx(abs(d) / 4.0, rel=1e-15)


def pin_scale_invariance(f=rmmc):
    rng = np.random.default_rng(2)
    M = rng.standard_normal((6, 4))
    Mn = M + 0.1 * rng.standard_normal((6, 4))
    ref = f(M, Mn)
    for c in (1e-6, 3.5, -2.0):
        assert f(c * M, c * Mn) == pytest.approx(ref, rel=1e-14)


def pin_zero_momentum(f=rmmc):
    Z = np.zeros((3, 3))
    assert f(Z, Z) == 0.0
    E = Z.copy()
    E[1, 2] = 1e-30
    assert f(Z, E) == float("inf")


def pin_full_rank_step_without_gradient(f=rmmc):
    rng = np.random.default_rng(3)
    for m, n, mu in ((12, 8, 0.9), (8, 12, 0.95), (10, 10, 0.5)):
        r = min(m, n)
        M = rng.standard_normal((m, n))
        Q = rng.standard_normal((n, r))
        o = dion_step(np.zeros((m, n)), np.zeros((m, n)), M, Q, mu, 0.01, 1e-8)
        assert np.allclose(o["M"], mu * M, rtol=0, atol=1e-12 * np.abs(M).max())
        assert f(M, o["M"]) == pytest.approx(1.0 - mu, rel=1e-11)


def pin_rank0_step(f=rmmc):
    rng = np.random.default_rng(4)
    M, G = rng.standard_normal((6, 9)), 1e-2 * rng.standard_normal((6, 9))
    o = dion_step(np.zeros((6, 9)), G, M, np.zeros((9, 0)), 0.95, 0.01, 1e-8)
    assert f(M, o["M"]) == pytest.approx(np.abs(G).max() / np.abs(M).max(), rel=1e-13)


PINS = [pin_no_change, pin_single_entry, pin_scale_invariance, pin_zero_momentum,
        pin_full_rank_step_without_gradient, pin_rank0_step]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def _scale_by_new(M, Mn):
    return float(np.max(np.abs(Mn - M)) / np.max(np.abs(Mn)))


def _elementwise_relative(M, Mn):
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.abs(Mn - M) / np.abs(M)
    return float(np.nanmax(q))


def _frobenius(M, Mn):
    return float(np.linalg.norm(Mn - M) / np.linalg.norm(M))


@pytest.mark.parametrize("bad", [_scale_by_new, _elementwise_relative, _frobenius])
def test_planted_mistake_is_caught(bad):
    caught = 0
    for pin in PINS:
        try:
            pin(bad)
        except (AssertionError, FloatingPointError, ZeroDivisionError):
            caught += 1
    assert caught > 0, f"{bad.__name__} passed every pin"
