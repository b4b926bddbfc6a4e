"""fp64 CPU oracle of the multi-power-iteration estimate of a largest eigenvalue.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, calls or links this
file; only the tests and the benchmark's CPU-baseline leg do.  It shares no
code with the GPU path.

Source: the DASH summary (gist.science), "Methodologie", 2. "Efficiënte
Inverse-Root Solvers", the item on multi-power-iteration scaling, and the same
item under "Belangrijkste Bijdragen": the spectral radius lambda_max of a
symmetric matrix is estimated by power iteration run in parallel from a pool of
start vectors (at most 32), and it replaces the Frobenius norm as the scale of
the matrix, which overestimates it.  In the Dion step the same role falls to the
shift of shifted CholeskyQR, which the plain form scales by trace(W) = ||P0||_F^2.

What is computed, for a symmetric positive semi-definite W (r x r) and a pool
V0 = [v_1 ... v_k] of start vectors:

    for each pool vector, t times:   v <- W v / ||W v||
    lambda_hat = max over the pool of the Rayleigh quotient  v^T W v / v^T v

Readings (each also listed in the design notes): the pages fix neither the
iteration count nor how the pool is combined; the estimate is the largest of the
pool's Rayleigh quotients, each taken after t normalized products (t + 1 products
in all).  A vector that W maps to zero contributes 0.  The pages' version runs in
half precision; this oracle is fp64, and the start vectors are inputs.

Pins: tests/test_spectral_pins.py checks this against closed forms and LAPACK's
symmetric eigenvalues (the estimate never exceeds lambda_max; it is exact for
rank-one and diagonal matrices; its error falls as (lambda_2 / lambda_1)^(2t) for
a start vector with no component outside the top two eigenvectors).
"""
from __future__ import annotations

import numpy as np


def power_iterate(W: np.ndarray, V0: np.ndarray, iters: int) -> np.ndarray:
    """The pool after ``iters`` normalized products: each column v <- W v / ||W v||.
    A column that W maps to zero stays zero."""
    V = np.array(V0, dtype=np.float64, copy=True)
    W = np.asarray(W, dtype=np.float64)
    for _ in range(iters):
        V = W @ V
        norms = np.linalg.norm(V, axis=0)
        V = np.divide(V, norms, out=np.zeros_like(V), where=norms > 0)
    return V


def rayleigh_quotients(W: np.ndarray, V: np.ndarray) -> np.ndarray:
    """v^T W v / v^T v for each column (0 for a zero column)."""
    W = np.asarray(W, dtype=np.float64)
    num = np.einsum("ij,ij->j", V, W @ V)
    den = np.einsum("ij,ij->j", V, V)
    return np.divide(num, den, out=np.zeros_like(num), where=den > 0)


def lambda_max_estimate(W: np.ndarray, V0: np.ndarray, iters: int) -> float:
    """Multi-power-iteration estimate of the largest eigenvalue of the symmetric PSD W."""
    if iters < 0:
        raise ValueError("iters >= 0")
    V0 = np.asarray(V0, dtype=np.float64)
    if V0.ndim != 2 or V0.shape[0] != np.asarray(W).shape[0] or V0.shape[1] < 1:
        raise ValueError("V0 is r x k with k >= 1")
    return float(rayleigh_quotients(W, power_iterate(W, V0, iters)).max())


def lambda_max_batched(W: np.ndarray, V0: np.ndarray, iters: int) -> np.ndarray:
    """``lambda_max_estimate`` over a stack: W [b, r, r], V0 [b, r, k]."""
    return np.array([lambda_max_estimate(W[i], V0[i], iters) for i in range(W.shape[0])])
