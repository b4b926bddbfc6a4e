"""50-digit reference of one Dion step for tiny inputs — TEST INFRASTRUCTURE ONLY.

An independent second implementation used to pin the fp64 oracle: every
product is formed in mpmath at ``dps`` decimal digits, and the orthonormal
factor comes from modified Gram-Schmidt (a different algorithm from the fp64
oracle's Householder QR; both give the unique Q-factor with a positive
diagonal when P0 has full column rank).  Steps and readings as in
``dion_oracle`` ("Dion e la fine del monopolio di Adam negli optimizer AI
distribuiti", rivista.ai: error feedback, power iteration, QR).
Pure-Python loops: meant for matrices of a few dozen entries.
"""
from __future__ import annotations

import mpmath as mp
import numpy as np


def _mat(a) -> list:
    a = np.asarray(a, dtype=np.float64)
    return [[mp.mpf(float(v)) for v in row] for row in a]


def _matmul(A, B):
    n_inner = len(B)
    return [[mp.fsum(A[i][k] * B[k][j] for k in range(n_inner)) for j in range(len(B[0]))]
            for i in range(len(A))]


def _t(A):
    return [list(col) for col in zip(*A)]


def mgs_qr(P0):
    """Modified Gram-Schmidt on the columns of P0 (list of rows): returns (P, T)."""
    m, r = len(P0), len(P0[0])
    V = [[P0[i][j] for i in range(m)] for j in range(r)]   # columns
    Pc, T = [], [[mp.mpf(0)] * r for _ in range(r)]
    for j in range(r):
        v = list(V[j])
        for i in range(j):
            t = mp.fsum(Pc[i][k] * v[k] for k in range(m))
            T[i][j] = t
            v = [v[k] - t * Pc[i][k] for k in range(m)]
        nrm = mp.sqrt(mp.fsum(x * x for x in v))
        T[j][j] = nrm
        Pc.append([x / nrm for x in v])
    P = [[Pc[j][i] for j in range(r)] for i in range(m)]
    return P, T


def dion_step_mp(X, G, M, Q, mu, lr, eps, dps: int = 50) -> dict:
    """One Dion step at ``dps`` digits; returns fp64 numpy arrays (rounded once at the end)."""
    with mp.workdps(dps):
        Xm, Gm, Mm, Qm = _mat(X), _mat(G), _mat(M), _mat(Q)
        m, n = len(Xm), len(Xm[0])
        r = len(Qm[0])
        B = [[Mm[i][j] + Gm[i][j] for j in range(n)] for i in range(m)]
        P0 = _matmul(B, Qm)
        P, T = mgs_qr(P0)
        R = _matmul(_t(B), P)
        PRt = _matmul(P, _t(R))
        one_minus_mu = 1 - mp.mpf(float(mu))
        Mn = [[B[i][j] - one_minus_mu * PRt[i][j] for j in range(n)] for i in range(m)]
        norms = [mp.sqrt(mp.fsum(R[i][j] ** 2 for i in range(n))) for j in range(r)]
        Qn = [[R[i][j] / (norms[j] + mp.mpf(float(eps))) for j in range(r)] for i in range(n)]
        s = mp.sqrt(mp.mpf(m) / n)
        PQt = _matmul(P, _t(Qn))
        lr_s = mp.mpf(float(lr)) * s
        Xn = [[Xm[i][j] - lr_s * PQt[i][j] for j in range(n)] for i in range(m)]

        def f(A):
            return np.array([[float(v) for v in row] for row in A], dtype=np.float64)

        return dict(X=f(Xn), M=f(Mn), Q=f(Qn), P=f(P), T=f(T), R=f(R), B=f(B), P0=f(P0), PQ=f(PQt))
