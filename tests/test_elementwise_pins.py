"""Pins of the element-wise oracle (AdamW, Lion) against closed forms.

The pages name AdamW and Lion for the parameters Dion does not take (rivista.ai,
the paragraph beginning "Tecnicamente") without printing their rules, so the
pins are properties the published rules fix, none of them a retyping of the
update:

  AdamW  first step from zero moments: the move is lr * g / (|g| + eps) whatever the
         betas (the bias corrections cancel exactly), and with decay the decoupled rule
         gives theta (1 - lr wd) - lr g / (|g| + eps), the decay taken on the weight as it
         was before the step; under a constant gradient every
         later step moves by the same amount (the corrected moments stay g and g^2);
         a zero gradient from zero moments only decays; the moments are geometric
         blends with weights (1 - beta)
  Lion   every coordinate moves by exactly lr (or 0 where the blend is 0) besides the
         decay, in the direction opposite the sign of beta1 m + (1 - beta1) g; at
         beta1 = 0 the direction is sign(g); the momentum after k steps of a constant
         gradient is g (1 - beta2^k) from zero

The planted-mistake tests patch a mistake into a copy of the oracle (on the CPU) and
check that a pin fails for each.
"""
import numpy as np
import pytest

import oracle.elementwise_oracle as E


def _draw(n, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(n), rng.standard_normal(n) * 1e-2


def pin_adamw_first_step(adamw=E.adamw_step):
    theta, g = _draw(257, 1)
    for b1, b2 in ((0.9, 0.999), (0.5, 0.9), (0.0, 0.0)):
        lr, eps, wd = 1e-3, 1e-8, 0.0
        th, m, v = adamw(theta, g, np.zeros_like(g), np.zeros_like(g), 1, lr, b1, b2, eps, wd)
        want = theta - lr * g / (np.abs(g) + eps)
        assert np.allclose(th, want, rtol=0, atol=1e-15), (b1, b2)
        assert np.allclose(m, (1 - b1) * g, rtol=1e-15, atol=0)
        assert np.allclose(v, (1 - b2) * g * g, rtol=1e-15, atol=0)


def pin_adamw_constant_gradient(adamw=E.adamw_step):
    theta, g = _draw(64, 2)
    lr, b1, b2, eps = 1e-2, 0.9, 0.99, 1e-8
    th, m, v = theta.copy(), np.zeros_like(g), np.zeros_like(g)
    for t in range(1, 9):
        prev = th
        th, m, v = adamw(th, g, m, v, t, lr, b1, b2, eps, 0.0)
        assert np.allclose(prev - th, lr * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-16), t
        assert np.allclose(m, g * (1 - b1 ** t), rtol=1e-12, atol=0), t
        assert np.allclose(v, g * g * (1 - b2 ** t), rtol=1e-12, atol=0), t


def pin_adamw_decay_only(adamw=E.adamw_step):
    theta, _ = _draw(33, 3)
    z = np.zeros_like(theta)
    th, m, v = adamw(theta, z, z, z, 1, 0.1, 0.9, 0.999, 1e-8, 0.5)
    assert np.array_equal(th, theta * (1 - 0.1 * 0.5)) and not m.any() and not v.any()


def pin_adamw_first_step_with_decay(adamw=E.adamw_step):
    """Decay and gradient both non-zero: the decoupled decay multiplies the weight as it was
    before the step, so step 1 from zero moments lands on theta (1 - lr wd) - lr g / (|g| + eps);
    decaying the stepped weight instead is off by lr wd times the move."""
    theta, g = _draw(129, 7)
    for lr, wd in ((0.1, 0.5), (1e-3, 0.1)):
        th, m, v = adamw(theta, g, np.zeros_like(g), np.zeros_like(g), 1, lr, 0.9, 0.999, 1e-8, wd)
        want = theta * (1 - lr * wd) - lr * g / (np.abs(g) + 1e-8)
        assert np.allclose(th, want, rtol=0, atol=1e-15), (lr, wd)


def pin_lion_unit_moves(lion=E.lion_step):
    theta, g = _draw(301, 4)
    g[::7] = 0.0
    rng = np.random.default_rng(5)
    m = rng.standard_normal(301) * 1e-2
    m[::7] = 0.0
    lr, b1, b2, wd = 3e-4, 0.9, 0.99, 0.1
    th, m2 = lion(theta, g, m, lr, b1, b2, wd)
    move = theta * (1 - lr * wd) - th
    blend = b1 * m + (1 - b1) * g
    assert np.allclose(np.abs(move[blend != 0]), lr, rtol=1e-12, atol=0)
    assert np.all(move[blend == 0] == 0)
    assert np.all(np.sign(move) == np.sign(blend))
    # beta1 = 0: the direction is sign(g)
    th0, _ = lion(theta, g, m, lr, 0.0, b2, 0.0)
    assert np.allclose(theta - th0, lr * np.sign(g), rtol=1e-12, atol=0)


def pin_lion_momentum(lion=E.lion_step):
    theta, g = _draw(40, 6)
    m = np.zeros_like(g)
    b2 = 0.95
    for k in range(1, 7):
        theta, m = lion(theta, g, m, 1e-3, 0.9, b2, 0.0)
        assert np.allclose(m, g * (1 - b2 ** k), rtol=1e-12, atol=0), k


PINS = [pin_adamw_first_step, pin_adamw_first_step_with_decay, pin_adamw_constant_gradient, pin_adamw_decay_only,
        pin_lion_unit_moves, pin_lion_momentum]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# planted mistakes: each must fail at least one pin
def _adamw_no_bias_correction(theta, g, m, v, t, lr, b1, b2, eps, wd):
    theta = theta * (1 - lr * wd)
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    return theta - lr * m / (np.sqrt(v) + eps), m, v


def _adamw_coupled_decay(theta, g, m, v, t, lr, b1, b2, eps, wd):
    return E.adamw_step(theta, g + wd * theta, m, v, t, lr, b1, b2, eps, 0.0)


def _adamw_swapped_betas(theta, g, m, v, t, lr, b1, b2, eps, wd):
    return E.adamw_step(theta, g, m, v, t, lr, b2, b1, eps, wd)


def _adamw_decay_after_step(theta, g, m, v, t, lr, b1, b2, eps, wd):
    th, m2, v2 = E.adamw_step(theta, g, m, v, t, lr, b1, b2, eps, 0.0)
    return th * (1 - lr * wd), m2, v2


def _lion_momentum_direction(theta, g, m, lr, b1, b2, wd):
    theta2, m2 = E.lion_step(theta, g, m, lr, b1, b2, wd)
    return theta * (1 - lr * wd) - lr * np.sign(m2), m2


def _lion_swapped_betas(theta, g, m, lr, b1, b2, wd):
    return E.lion_step(theta, g, m, lr, b2, b1, wd)


@pytest.mark.parametrize("bad,pins", [
    (_adamw_no_bias_correction, [pin_adamw_first_step, pin_adamw_constant_gradient]),
    (_adamw_coupled_decay, [pin_adamw_decay_only]),
    (_adamw_swapped_betas, [pin_adamw_first_step, pin_adamw_constant_gradient]),
    (_adamw_decay_after_step, [pin_adamw_first_step_with_decay]),
    (_lion_momentum_direction, [pin_lion_unit_moves]),
    (_lion_swapped_betas, [pin_lion_momentum, pin_lion_unit_moves]),
])
def test_planted_mistake_is_caught(bad, pins):
    caught = 0
    for pin in pins:
        try:
            pin(bad)
        except AssertionError:
            caught += 1
    assert caught > 0, f"{bad.__name__} passed every pin"
