"""fp64 CPU oracle of the element-wise optimizers for the parameters Dion does not take.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, calls or links this
file; only the tests and the benchmark's CPU-baseline leg do.  It shares no
code with the GPU path.

Source: "Dion e la fine del monopolio di Adam negli optimizer AI distribuiti"
(rivista.ai), the paragraph beginning "Tecnicamente": Dion takes the 2-D
parameters only, and biases and 1-D weights are left to optimizers such as
AdamW or Lion.  The pages name the two optimizers without writing their update
rules, so these are the published algorithms, in their plainest form (each
reading also listed in the design notes):

  AdamW (Adam with decoupled weight decay), step t = 1, 2, ...:
      theta <- theta * (1 - lr * wd)
      m     <- beta1 * m + (1 - beta1) * g
      v     <- beta2 * v + (1 - beta2) * g^2
      theta <- theta - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)

  Lion (sign of an interpolated momentum, decoupled weight decay):
      c     <- beta1 * m + (1 - beta1) * g
      theta <- theta * (1 - lr * wd) - lr * sign(c)          sign(0) = 0
      m     <- beta2 * m + (1 - beta2) * g

Inputs are the exact fp64 upcasts of the stored values; outputs are fp64 and
are compared before any rounding to storage.

Pins: tests/test_oracle_pins.py checks these functions against closed forms
that do not retype them (the first AdamW step is lr * sign-like and does not
depend on the betas; under a constant gradient the bias-corrected moments are
exact; Lion moves every coordinate by exactly lr or 0, and its momentum is a
fixed geometric blend).
"""
from __future__ import annotations

import numpy as np


def adamw_step(theta, g, m, v, t: int, lr: float, beta1: float, beta2: float, eps: float, wd: float):
    """One AdamW step; returns (theta', m', v') in fp64."""
    theta = np.asarray(theta, np.float64)
    g = np.asarray(g, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    if t < 1:
        raise ValueError("AdamW steps count from 1")
    theta = theta * (1.0 - lr * wd)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    theta = theta - lr * mhat / (np.sqrt(vhat) + eps)
    return theta, m, v


def lion_step(theta, g, m, lr: float, beta1: float, beta2: float, wd: float):
    """One Lion step; returns (theta', m') in fp64."""
    theta = np.asarray(theta, np.float64)
    g = np.asarray(g, np.float64)
    m = np.asarray(m, np.float64)
    c = beta1 * m + (1.0 - beta1) * g
    theta = theta * (1.0 - lr * wd) - lr * np.sign(c)
    m = beta2 * m + (1.0 - beta2) * g
    return theta, m
