"""Shared test plumbing: run the GPU step on workload inputs and compare with the oracle.

Parity is judged teacher-forced: every step starts the oracle from the exact
state bits the GPU stored after the previous step, with the same G_t.
"""
from __future__ import annotations

import numpy as np

import workloads as W
from oracle import dion_step

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def tol_for(wl) -> float:
    return TOL_BF16 if wl.x_dtype == "bf16" else TOL_F32


def rel(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    d = np.linalg.norm(a - b)
    return float(d / nb) if nb > 0 else float(d)


def to_torch(a: np.ndarray, device):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_numpy(t) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def compare_step(wl, pre, post, G, rank, idx=None):
    """Per-matrix errors of one GPU step against the oracle started from `pre`.

    pre/post: dicts of host arrays X, M, Q (+ post P).  Returns a list of dicts.
    """
    out = []
    b = pre["X"].shape[0]
    for i in (range(b) if idx is None else idx):
        o = dion_step(W.to_f64(pre["X"][i], wl.x_dtype), W.to_f64(G[i], wl.g_dtype),
                      pre["M"][i].astype(np.float64), pre["Q"][i].astype(np.float64), wl.mu, wl.lr, wl.eps)
        e = {"M": rel(post["M"][i].astype(np.float64), o["M"]),
             "X": rel(W.to_f64(post["X"][i], wl.x_dtype), o["X"])}
        if rank:
            P = post["P"][i].astype(np.float64)
            Qn = post["Q"][i].astype(np.float64)
            e["PQ"] = rel(P @ Qn.T, o["P"] @ o["Q"].T)
            e["Q"] = rel(Qn, o["Q"])
            e["orth"] = float(np.abs(P.T @ P - np.eye(rank)).max())
        e["rank_deficient"] = bool(o["rank_deficient"])
        out.append(e)
    return out
