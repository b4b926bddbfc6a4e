"""fp64 CPU oracle of one Dion optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, calls or links
this file; only the tests, the package's smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the GPU path: the GPU path
orthonormalizes by Cholesky-based QR, this oracle by LAPACK Householder QR.

What is computed (one step, per matrix X of shape m x n, rank r):

    B  = M + G                                   error-feedback buffer
    P0 = B Q                                     one warm-started power-iteration step
    P  = Q-factor of the thin QR of P0           orthonormal m x r, unpivoted, diag(T) > 0
    R  = B^T P
    M' = B - (1 - mu) P R^T                      the residual the low-rank update missed
    Q' = R / (||r_j||_2 + eps)   column-wise     warm start for the next step
    X' = X - lr * sqrt(m / n) * P Q'^T

Sources, by page title and passage:
  * "Dion e la fine del monopolio di Adam negli optimizer AI distribuiti"
    (rivista.ai): orthonormalize only the first r singular directions (the
    paragraph introducing rank as a scaling dimension); error feedback keeps the
    full-versus-low-rank difference and re-injects it in later updates (the
    paragraph on FSDP traffic); amortized power iteration with QR and Cholesky
    replaces Newton-Schulz, and only 2-D parameters go to Dion (the paragraph
    beginning "Tecnicamente").  The title line names the method "Dion:
    Distributed Orthonormalized Updates".
  * "DeMuon" summary (gist.science, "Metodología", "Ortogonalización de
    Matrices"): msgn(B) = U V^T, the full-rank limit used as a pin.
  * "DASH" summary (gist.science, "Methodologie", 3-D tensor stacking): the
    step is batched over stacks of same-shape matrices.

Readings where the pages are silent (each also listed in the design notes):
  * s = sqrt(m / n) for X of shape m x n;
  * eps only in the column normalization, as ||r_j|| + eps;
  * "orthonormalize" = Q-factor of the unpivoted thin QR in column order
    with a positive diagonal;
  * every product is formed in fp64 from the exact upcast of the stored
    (fp32 or bf16) inputs; outputs are compared before any rounding.

Pins: tests/test_oracle_pins.py checks every function here against closed
forms, textbook routines, brute force and 50-digit arithmetic.  Multi-step
trajectories have no independent pin: parity unpinned beyond the per-step
pins (the pages print no worked example).
"""
from __future__ import annotations

import math

import numpy as np

# Relative diagonal threshold under which the QR of P0 is called rank deficient:
# the Q-factor is then not unique and only invariants are compared.
RANK_DEFICIENT_RTOL = 1e-13


def accumulate(M: np.ndarray, G: np.ndarray) -> np.ndarray:
    """Error-feedback buffer B = M + G (exact for fp32/bf16 inputs upcast to fp64)."""
    return M + G


def power_step(B: np.ndarray, Q: np.ndarray) -> np.ndarray:
    """One warm-started power-iteration step P0 = B Q."""
    return B @ Q


def thin_qr_positive(P0: np.ndarray):
    """Unpivoted thin QR with a positive diagonal: returns (P, T) with P0 = P T.

    LAPACK Householder (dgeqrf/dorgqr) through numpy, then the sign of every
    column of P (and row of T) flipped so that diag(T) > 0, which makes the
    Q-factor unique when P0 has full column rank.
    """
    P, T = np.linalg.qr(np.asarray(P0, dtype=np.float64), mode="reduced")
    d = np.sign(np.diag(T))
    d[d == 0] = 1.0
    return P * d[None, :], T * d[:, None]


def project_back(B: np.ndarray, P: np.ndarray) -> np.ndarray:
    """R = B^T P: the right factor of the rank-r approximation P R^T of B."""
    return B.T @ P


def error_feedback(B: np.ndarray, P: np.ndarray, R: np.ndarray, mu: float) -> np.ndarray:
    """M' = B - (1 - mu) P R^T: what the low-rank update did not take stays in M."""
    return B - (1.0 - mu) * (P @ R.T)


def column_normalize(R: np.ndarray, eps: float) -> np.ndarray:
    """Q' with columns q_j = r_j / (||r_j||_2 + eps)."""
    return R / (np.linalg.norm(R, axis=0, keepdims=True) + eps)


def update_scale(m: int, n: int) -> float:
    """s in X' = X - lr * s * P Q'^T: sqrt(m / n) for an m x n weight."""
    return math.sqrt(m / n)


def weight_update(X: np.ndarray, P: np.ndarray, Qn: np.ndarray, lr: float, s: float) -> np.ndarray:
    """X' = X - lr * s * P Q'^T."""
    return X - lr * s * (P @ Qn.T)


def dion_step(X: np.ndarray, G: np.ndarray, M: np.ndarray, Q: np.ndarray,
              mu: float, lr: float, eps: float) -> dict:
    """One Dion step of one m x n matrix, every operand already in fp64.

    ``Q`` is n x r (r may be 0).  Returns a dict with the new state
    ``X, M, Q`` and the intermediates ``B, P0, P, T, R``, plus
    ``rank_deficient`` (True when the Q-factor of P0 is not unique).
    The steps run in the method's order; each is a module-level function so
    that the pin tests can plant a mistake in one of them.
    """
    X = np.asarray(X, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    m, n = X.shape
    r = Q.shape[1]
    B = accumulate(M, G)
    if r == 0:
        z = np.zeros((m, 0))
        return dict(X=X.copy(), M=B, Q=Q.copy(), B=B, P0=z, P=z, T=np.zeros((0, 0)),
                    R=np.zeros((n, 0)), rank_deficient=False)
    P0 = power_step(B, Q)
    P, T = thin_qr_positive(P0)
    dT = np.abs(np.diag(T))
    rank_deficient = bool(dT.min() <= RANK_DEFICIENT_RTOL * dT.max())
    R = project_back(B, P)
    M_new = error_feedback(B, P, R, mu)
    Q_new = column_normalize(R, eps)
    X_new = weight_update(X, P, Q_new, lr, update_scale(m, n))
    return dict(X=X_new, M=M_new, Q=Q_new, B=B, P0=P0, P=P, T=T, R=R,
                rank_deficient=rank_deficient)


def dion_step_batched(X: np.ndarray, G: np.ndarray, M: np.ndarray, Q: np.ndarray,
                      mu: float, lr: float, eps: float) -> dict:
    """dion_step over a stack [b, m, n] (Q is [b, n, r]); results stacked likewise."""
    outs = [dion_step(X[i], G[i], M[i], Q[i], mu, lr, eps) for i in range(X.shape[0])]
    keys = ("X", "M", "Q", "B", "P0", "P", "T", "R")
    res = {k: np.stack([o[k] for o in outs]) if outs else None for k in keys}
    res["rank_deficient"] = np.array([o["rank_deficient"] for o in outs], dtype=bool)
    return res
