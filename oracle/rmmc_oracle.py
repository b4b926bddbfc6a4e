"""fp64 CPU oracle of the Relative Maximum Momentum Change (RMMC) of one Dion step.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, calls or links this
file; only the tests do.  It shares no code with the GPU path.

Source: "CurvaDion: Curvature-Adaptive Distributed Orthonormalization"
(mlsanity.com), "Abstract (arXiv)": CurvaDion detects high-curvature regions,
where workers must synchronize, with a statistic named Relative Maximum Momentum
Change; it is built from the momentum dynamics the optimizer already computes,
serves as a proxy for directional curvature, and costs O(d) operations per layer.
The page gives the name and the cost, not the formula.

Reading (also listed in the design notes), taken from the name: per layer (one
matrix of the stack), the largest absolute change of a momentum entry over one
step, relative to the largest absolute momentum entry before the step,

    RMMC = max_ij |M'_ij - M_ij| / max_ij |M_ij|,

with M the momentum entering the step and M' the one the step leaves (in Dion's
error feedback M' = M + G - (1 - mu) P R^T).  Both maxima are one pass over the
layer's entries (O(d)).  Where max |M| = 0 (the first step from M = 0) the value
is 0 if M' = M as well and +inf otherwise: a change from zero momentum counts as
unboundedly large.

Pins: tests/test_rmmc_pins.py (closed forms on constructed momenta, invariance
under a common scale, and the full-rank Dion step with G = 0, where M' = mu M
exactly and RMMC = 1 - mu).
"""
from __future__ import annotations

import numpy as np


def rmmc(M_old: np.ndarray, M_new: np.ndarray) -> float:
    """max |M_new - M_old| / max |M_old| over all entries (see the module docstring)."""
    M_old = np.asarray(M_old, dtype=np.float64)
    M_new = np.asarray(M_new, dtype=np.float64)
    change = float(np.max(np.abs(M_new - M_old))) if M_old.size else 0.0
    scale = float(np.max(np.abs(M_old))) if M_old.size else 0.0
    if scale == 0.0:
        return 0.0 if change == 0.0 else float("inf")
    return change / scale
