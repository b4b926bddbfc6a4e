"""Shared test plumbing: run the GPU step on workload inputs and compare with the oracle.

Parity is judged teacher-forced: every step starts the oracle from the exact
state bits the GPU stored after the previous step, with the same G_t.

Besides the relative Frobenius errors of P Q'^T, M' and X' (M' and X' are dominated by
the unchanged B and X, so those two alone would let a wrong update through), every step
checks the updates themselves:
  dM   rel(B - M'_gpu, B - fl32(M'_oracle))   with B = M + G exact in fp64;
  dX   rel(X - X'_gpu, X - fl32(X'_oracle))   for fp32 weights;
  Xband  element-wise: X'_gpu is the stored rounding of a value within b_ij of
         X - lr s (P Q'^T)_ij formed in fp64 from the GPU's own P and Q', where
         b_ij = lr s gamma (|P| |Q'|^T)_ij + 2^-23 |X'|: gamma bounds the rounding of
         the weight pass's product (see update_gamma) and the last term its fp32
         rounding.  No element may fall outside (bf16: outside the roundings of the
         interval's ends).  Together with the P Q'^T check against the oracle this pins
         X' = X - lr s P Q'^T element by element.
"""
from __future__ import annotations

import math

import numpy as np

import workloads as W
from oracle import dion_step

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def tol_for(wl) -> float:
    return TOL_BF16 if wl.x_dtype == "bf16" else TOL_F32


def update_gamma(rank: int, arith: str = "split6") -> float:
    """Relative bound of the weight pass's product P Q'^T against (|P| |Q'|^T)_ij.

    split6: fp32 operands split exactly into three bf16 parts, six of the nine part
    products kept (the three dropped ones are below 2^-24 |a||b| each: at most 2.1 u),
    exact bf16 x bf16 products accumulated in fp32 (at most 6 r additions, 6 r u), plus
    the fp32 rounding of lr s (u).  split3: each operand split into two bf16 parts, a = h + l + e
    with |l| <= 2^-8 (1 + 2^-8) |a| and |e| <= 2^-16 |a|; the kept products h h, h l, l h drop
    l l and the e terms, together below 3.01 * 2^-16 |a||b|, then 3 r fp32 additions and lr s.
    bf16: both operands rounded once to bf16 (2 * 2^-8), accumulated in fp32 (r u), plus lr s
    (u).  u = 2^-24."""
    u = 2.0 ** -24
    if arith == "split6":
        return (6 * rank + 4) * u
    if arith == "split3":
        return 3.01 * 2.0 ** -16 + (3 * rank + 2) * u
    if arith == "bf16":
        return 2.0 * 2.0 ** -8 + 2.0 ** -16 + (rank + 2) * u
    raise ValueError(arith)


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


def _f32(a: np.ndarray) -> np.ndarray:
    return a.astype(np.float32).astype(np.float64)


def _bf16_value(a64: np.ndarray) -> np.ndarray:
    """Value of RNE_bf16(fl32(a)) in fp64 (monotone in a)."""
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(a64.astype(np.float32))).astype(np.float64)


def xband_violations(X0: np.ndarray, Xg: np.ndarray, P: np.ndarray, Qn: np.ndarray, lr_s: float, gamma: float,
                     x_dtype: str) -> int:
    """Elements of X'_gpu that no rounding of a value within the band around X - lr_s P Q'^T
    explains (see the module docstring).  All arrays fp64 except the stored X'_gpu values."""
    Xe = X0 - lr_s * (P @ Qn.T)
    b = lr_s * gamma * (np.abs(P) @ np.abs(Qn).T) + 2.0 ** -23 * np.abs(Xe) + 1e-300
    lo, hi = Xe - b, Xe + b
    if x_dtype == "bf16":
        lo, hi = _bf16_value(lo), _bf16_value(hi)
    return int(np.count_nonzero((Xg < lo) | (Xg > hi)))


def arith_for(wl, options: int = 0) -> str:
    """The weight pass's arithmetic: with the exact-products option the fp32-accurate six-product
    split; otherwise plain bf16 products for bf16 weights, the two-part split for fp32 ones."""
    from rank_orthonormalized_optimizer_amd._lib import OPT_EXACT_PRODUCTS
    if options & OPT_EXACT_PRODUCTS:
        return "split6"
    return "bf16" if wl.x_dtype == "bf16" else "split3"


def compare_step(wl, pre, post, G, rank, idx=None, arith: str | None = None):
    """Per-matrix errors of one GPU step against the oracle started from `pre`.

    pre/post: dicts of host arrays X, M, Q (+ post P).  ``arith``: the weight pass's arithmetic
    ("split6", "split3" or "bf16"; default: arith_for(wl)).  Returns a list of dicts.
    """
    if arith is None:
        arith = arith_for(wl)
    out = []
    b = pre["X"].shape[0]
    m, n = pre["X"].shape[1], pre["X"].shape[2]
    lr_s = float(np.float32(wl.lr * math.sqrt(m / n)))
    for i in (range(b) if idx is None else idx):
        X0 = W.to_f64(pre["X"][i], wl.x_dtype)
        o = dion_step(X0, W.to_f64(G[i], wl.g_dtype), pre["M"][i].astype(np.float64),
                      pre["Q"][i].astype(np.float64), wl.mu, wl.lr, wl.eps)
        Mg = post["M"][i].astype(np.float64)
        Xg = W.to_f64(post["X"][i], wl.x_dtype)
        e = {"M": rel(Mg, o["M"]), "X": rel(Xg, o["X"])}
        if rank:
            B = o["B"]
            e["dM"] = rel(B - Mg, B - _f32(o["M"]))
            if wl.x_dtype == "f32":
                e["dX"] = rel(X0 - Xg, X0 - _f32(o["X"]))
            else:
                e["X_rne_match"] = float(np.mean(Xg == _bf16_value(o["X"])))
            P = post["P"][i].astype(np.float64)
            Qn = post["Q"][i].astype(np.float64)
            e["PQ"] = rel(P @ Qn.T, o["P"] @ o["Q"].T)
            e["Q"] = rel(Qn, o["Q"])
            e["orth"] = float(np.abs(P.T @ P - np.eye(rank)).max())
            e["Xband"] = xband_violations(X0, Xg, P, Qn, lr_s, update_gamma(rank, arith), wl.x_dtype)
        e["rank_deficient"] = bool(o["rank_deficient"])
        out.append(e)
    return out


# keys judged against the workload's tolerance, and the count that must be zero
TOL_KEYS = ("PQ", "M", "X", "dM", "dX")


def check_errs(e: dict, tol: float, where: str = "") -> None:
    for k in TOL_KEYS:
        if k in e:
            assert e[k] <= tol, f"{where}: {k} rel err {e[k]:.3e} > {tol}"
    if "Xband" in e:
        assert e["Xband"] == 0, f"{where}: {e['Xband']} elements of X' outside the update band"
