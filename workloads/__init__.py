"""Seeded synthetic inputs for the Dion step.

This module is shared by the fp64 oracle's tests and by the GPU path's tests
and benchmark.  It holds the workload definitions and the random draws only:
none of the optimizer's arithmetic lives here.  Every value is drawn in fp64
from numpy's PCG64 and rounded once (round-to-nearest-even) to its storage type,
so both sides read identical bits.

The five workloads are stacks of same-shape 2-D weight matrices, the batching
unit used by the DASH page ("Batched Block Preconditioning", 3-D tensor
stacking); the shapes stand in for the models the pages train (a 2048-hidden
Llama on the DASH page's "Experimentele Resultaten", 10^8 to 10^9 parameter
models on the rivista.ai Dion page).  No dataset is read: gradients are
synthetic with the distributions listed per workload.

Stream keys: every array is drawn from
``Generator(PCG64(SeedSequence([seed, wid, group, matrix, step, tag, block])))``
so that any matrix (and any 1024-row block of it) can be regenerated alone.
"""
from __future__ import annotations

import math
import os
import sys
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

# stream tags
_T_X, _T_Q, _T_G, _T_U, _T_V, _T_NOISE, _T_SCALE = 0, 1, 2, 3, 4, 5, 6
_ROW_BLOCK = 1024


# ----------------------------------------------------------------------------
# bf16 storage helpers (encoding only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of a stored array (``dtype`` is 'f32' or 'bf16')."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def store(a64: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage type (f32 RNE, then bf16 RNE)."""
    f = a64.astype(np.float32)
    return f32_to_bf16_bits(f) if dtype == "bf16" else f


# ----------------------------------------------------------------------------
# workload definitions
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Group:
    """One stack of ``batch`` matrices of shape m x n, updated at rank ``rank``."""
    batch: int
    m: int
    n: int
    rank: int


@dataclass(frozen=True)
class Workload:
    wid: int                 # workload id (1..5), part of every stream key
    name: str
    groups: tuple
    mu: float
    lr: float = 0.01
    eps: float = 1e-8
    steps: int = 3
    x_dtype: str = "f32"     # storage type of X (and of G)
    grad: str = "gauss"      # gradient recipe, see make_grad
    grad_args: dict = field(default_factory=dict)

    @property
    def g_dtype(self) -> str:
        return self.x_dtype

    def with_groups(self, *groups: Group, name: str | None = None, steps: int | None = None) -> "Workload":
        return replace(self, groups=tuple(groups), name=name or self.name + "-small",
                       steps=self.steps if steps is None else steps)

    def params(self) -> int:
        return sum(g.batch * g.m * g.n for g in self.groups)


def _frac_rank(m: int, n: int, num: int, den: int) -> int:
    return (num * min(m, n)) // den


WORKLOADS = {
    1: Workload(1, "single-256x512-r32", (Group(1, 256, 512, 32),), mu=0.95, steps=10,
                grad="gauss", grad_args={"std": 1e-2}),
    2: Workload(2, "attn-24x1024x1024-r256", (Group(24, 1024, 1024, 256),), mu=0.95, steps=5,
                grad="lowrank_noise", grad_args={"k": 16, "noise_std": 1e-3}),
    3: Workload(3, "llama2048-bf16-r1/8",
                (Group(64, 2048, 2048, 256), Group(32, 5632, 2048, 256), Group(16, 2048, 5632, 256)),
                mu=0.95, steps=3, x_dtype="bf16",
                grad="loguniform_gauss", grad_args={"lo": 1e-5, "hi": 1e-2}),
    4: Workload(4, "mlp-8192x28672-r512", (Group(1, 8192, 28672, 512),), mu=0.95, steps=3,
                grad="student_t", grad_args={"nu": 3.0, "scale": 1e-3}),
    5: Workload(5, "fullrank-8x4096x4096", (Group(8, 4096, 4096, 4096),), mu=0.9, steps=3,
                grad="decaying_spectrum", grad_args={"decades": 6.0}),
}


def get(wid: int) -> Workload:
    return WORKLOADS[wid]


# Reduced-size versions with the same recipes, for CPU-speed parity tests.
# Shapes span several 64/128 tiles and leave ragged tails.
SMALL = {
    1: WORKLOADS[1].with_groups(Group(1, 256, 512, 32), name="single-256x512-r32", steps=4),
    2: WORKLOADS[2].with_groups(Group(3, 320, 288, 72), steps=3),
    3: WORKLOADS[3].with_groups(Group(2, 200, 136, 17), Group(2, 136, 200, 24), steps=2),
    4: WORKLOADS[4].with_groups(Group(1, 192, 1000, 40), steps=2),
    5: WORKLOADS[5].with_groups(Group(2, 160, 160, 160), steps=2),
}


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------
def _rng(seed: int, wid: int, gi: int, mi: int, step: int, tag: int, block: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, gi, mi, step, tag, block])))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_blocks(out: np.ndarray, fn, nthreads: int | None = None) -> None:
    """Run fn(mi, r0, r1) -> fp64 block for every matrix and 1024-row block, in threads."""
    b, m, _ = out.shape
    tasks = [(mi, r0, min(m, r0 + _ROW_BLOCK)) for mi in range(b) for r0 in range(0, m, _ROW_BLOCK)]

    def run(t):
        mi, r0, r1 = t
        out[mi, r0:r1] = fn(mi, r0, r1)

    with ThreadPoolExecutor(nthreads or _workers()) as ex:
        list(ex.map(run, tasks))


def make_state(wl: Workload, gi: int, seed: int = 0):
    """Initial (X, M, Q) of group ``gi``.

    X ~ N(0, 0.02^2) in the workload's storage type, M = 0 (fp32),
    Q = Gaussian n x r with each column scaled to unit norm (fp32).
    """
    g = wl.groups[gi]
    xdt = np.uint16 if wl.x_dtype == "bf16" else np.float32
    X = np.empty((g.batch, g.m, g.n), dtype=xdt)

    def xblock(mi, r0, r1):
        return store(0.02 * _rng(seed, wl.wid, gi, mi, 0, _T_X, r0 // _ROW_BLOCK).standard_normal((r1 - r0, g.n)),
                     wl.x_dtype)

    _fill_blocks(X, xblock)
    M = np.zeros((g.batch, g.m, g.n), dtype=np.float32)
    Q = np.empty((g.batch, g.n, g.rank), dtype=np.float32)
    for mi in range(g.batch):
        q = _rng(seed, wl.wid, gi, mi, 0, _T_Q).standard_normal((g.n, g.rank))
        if g.rank:
            q /= np.linalg.norm(q, axis=0, keepdims=True)
        Q[mi] = q.astype(np.float32)
    return X, M, Q


def _haar(rng: np.random.Generator, n: int) -> np.ndarray:
    z = rng.standard_normal((n, n))
    q, t = np.linalg.qr(z)
    return q * np.sign(np.diag(t))[None, :]


def make_grad(wl: Workload, gi: int, step: int, seed: int = 0) -> np.ndarray:
    """Gradient G_t of group ``gi`` at step ``step`` (1-based), fresh every step.

    Recipes (N(0, v) names a variance):
      gauss             G ~ N(0, std^2)
      lowrank_noise     G = U V^T + N(0, noise_std^2), U (m x k), V (n x k) ~ N(0, 1)
      loguniform_gauss  G = c_i N(0, 1), c_i ~ LogUniform(lo, hi) drawn once per matrix
      student_t         G = scale * t_nu
      decaying_spectrum G = U diag(10^(-decades i / n)) V^T, U, V Haar orthogonal
    """
    g = wl.groups[gi]
    a = wl.grad_args
    dt = wl.g_dtype
    out = np.empty((g.batch, g.m, g.n), dtype=np.uint16 if dt == "bf16" else np.float32)
    kind = wl.grad

    if kind == "gauss":
        def fn(mi, r0, r1):
            return store(a["std"] * _rng(seed, wl.wid, gi, mi, step, _T_G, r0 // _ROW_BLOCK)
                         .standard_normal((r1 - r0, g.n)), dt)
        _fill_blocks(out, fn)
    elif kind == "lowrank_noise":
        k = a["k"]
        UV = []
        for mi in range(g.batch):
            U = _rng(seed, wl.wid, gi, mi, step, _T_U).standard_normal((g.m, k))
            V = _rng(seed, wl.wid, gi, mi, step, _T_V).standard_normal((g.n, k))
            UV.append((U, V))

        def fn(mi, r0, r1):
            U, V = UV[mi]
            noise = _rng(seed, wl.wid, gi, mi, step, _T_NOISE, r0 // _ROW_BLOCK).standard_normal((r1 - r0, g.n))
            return store(U[r0:r1] @ V.T + a["noise_std"] * noise, dt)
        _fill_blocks(out, fn)
    elif kind == "loguniform_gauss":
        lo, hi = math.log(a["lo"]), math.log(a["hi"])
        scales = [math.exp(_rng(seed, wl.wid, gi, mi, 0, _T_SCALE).uniform(lo, hi)) for mi in range(g.batch)]

        def fn(mi, r0, r1):
            return store(scales[mi] * _rng(seed, wl.wid, gi, mi, step, _T_G, r0 // _ROW_BLOCK)
                         .standard_normal((r1 - r0, g.n)), dt)
        _fill_blocks(out, fn)
    elif kind == "student_t":
        def fn(mi, r0, r1):
            return store(a["scale"] * _rng(seed, wl.wid, gi, mi, step, _T_G, r0 // _ROW_BLOCK)
                         .standard_t(a["nu"], (r1 - r0, g.n)), dt)
        _fill_blocks(out, fn)
    elif kind == "decaying_spectrum":
        if g.m != g.n:
            raise ValueError("decaying_spectrum needs square matrices")
        n = g.n
        sig = 10.0 ** (-a["decades"] * np.arange(n) / n)

        # one matrix at a time: the QRs and the product already use every BLAS thread
        for mi in range(g.batch):
            if n >= 1024:
                print(f"[workloads] {wl.name} step {step}: Haar factors of matrix {mi + 1}/{g.batch}",
                      file=sys.stderr, flush=True)
            U = _haar(_rng(seed, wl.wid, gi, mi, step, _T_U), n)
            V = _haar(_rng(seed, wl.wid, gi, mi, step, _T_V), n)
            out[mi] = store((U * sig[None, :]) @ V.T, dt)
    else:
        raise ValueError(f"unknown gradient recipe {kind!r}")
    return out


# ----------------------------------------------------------------------------
# start vectors of the multi-power-iteration estimate (a counter-based stream)
# ----------------------------------------------------------------------------
_GOLDEN64 = 0x9E3779B97F4A7C15
_MASK64 = (1 << 64) - 1


def splitmix64(n: np.ndarray) -> np.ndarray:
    """Output number n (n >= 1) of SplitMix64 seeded with 0 (Steele, Lea and Flood, "Fast
    Splittable Pseudorandom Number Generators", 2014): the state n * 0x9E3779B97F4A7C15
    (mod 2^64) through the variant-13 finalizer.  Vectorized over uint64 counters."""
    z = np.asarray(n, dtype=np.uint64) * np.uint64(_GOLDEN64)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def splitmix_start_vectors(batch: int, r: int, k: int) -> np.ndarray:
    """The library's default start vectors of the lambda_max estimate, [batch, r, k] fp64:
    entry (b, i, j) is 2u - 1 with u the top 53 bits of SplitMix64 output b*r*k + i*k + j + 1
    over 2^53 (exact in fp64)."""
    idx = np.arange(batch * r * k, dtype=np.uint64) + np.uint64(1)
    with np.errstate(over="ignore"):
        z = splitmix64(idx)
    u = (z >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return (2.0 * u - 1.0).reshape(batch, r, k)


def psd_stack(batch: int, r: int, seed: int, kind: str = "gram", decades: float = 6.0) -> np.ndarray:
    """Symmetric PSD test matrices [batch, r, r] fp64: "gram" = A^T A with A (r + 8) x r Gaussian
    (a Gram matrix like P0^T P0), "spectrum" = U diag(10^(-decades i / r)) U^T with U Haar."""
    out = np.empty((batch, r, r))
    for b in range(batch):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, r, b, len(kind)])))
        if kind == "gram":
            A = rng.standard_normal((r + 8, r))
            out[b] = A.T @ A
        else:
            U = _haar(rng, r)
            out[b] = (U * 10.0 ** (-decades * np.arange(r) / r)) @ U.T
    return out


# ----------------------------------------------------------------------------
# the same recipes drawn on the GPU (benchmark inputs at full size)
# ----------------------------------------------------------------------------
# The benchmark needs the full-size inputs in HBM quickly; the workload-5 recipe alone costs two
# 4096^2 Haar QRs per matrix and step on the host.  These draw the same distributions with torch
# on the device (fp64, rounded once to the storage type, round-to-nearest-even), from a torch
# generator seeded per (seed, workload, group, step, tag).  They are not the host streams above:
# the reduced-size parity tests draw on the host; the full-size ones draw here and copy the
# sampled matrices back, so the oracle reads exactly the bits the GPU read.
def _torch_gen(device, *key):
    import torch
    s = np.random.SeedSequence([0x5EED, *key]).generate_state(1, np.uint64)[0]
    return torch.Generator(device=device).manual_seed(int(s) & ((1 << 63) - 1))


def _torch_store(a64, dtype: str):
    import torch
    f = a64.to(torch.float32)
    return f.to(torch.bfloat16) if dtype == "bf16" else f


def make_state_device(wl: Workload, gi: int, device, seed: int = 0):
    """Initial (X, M, Q) of group ``gi`` as device tensors, drawn on the device (see above)."""
    import torch
    g = wl.groups[gi]
    gen = _torch_gen(device, seed, wl.wid, gi, 0, _T_X)
    X = torch.empty((g.batch, g.m, g.n), dtype=torch.bfloat16 if wl.x_dtype == "bf16" else torch.float32,
                    device=device)
    for mi in range(g.batch):
        X[mi] = _torch_store(0.02 * torch.randn((g.m, g.n), generator=gen, device=device, dtype=torch.float64),
                             wl.x_dtype)
    M = torch.zeros((g.batch, g.m, g.n), dtype=torch.float32, device=device)
    gq = _torch_gen(device, seed, wl.wid, gi, 0, _T_Q)
    q = torch.randn((g.batch, g.n, g.rank), generator=gq, device=device, dtype=torch.float64)
    if g.rank:
        q /= torch.linalg.vector_norm(q, dim=1, keepdim=True)
    return X, M, q.to(torch.float32).contiguous()


def make_grad_device(wl: Workload, gi: int, step: int, device, seed: int = 0):
    """Gradient G_t of group ``gi`` as a device tensor: make_grad's recipe drawn on the device."""
    import torch
    g = wl.groups[gi]
    a = wl.grad_args
    dt = wl.g_dtype
    gen = _torch_gen(device, seed, wl.wid, gi, step, _T_G)
    out = torch.empty((g.batch, g.m, g.n), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device=device)

    def randn(*shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float64)

    kind = wl.grad
    if kind == "loguniform_gauss":
        gs = _torch_gen(device, seed, wl.wid, gi, 0, _T_SCALE)
        lo, hi = math.log(a["lo"]), math.log(a["hi"])
        scales = torch.exp(lo + (hi - lo) * torch.rand((g.batch,), generator=gs, device=device,
                                                        dtype=torch.float64)).tolist()
    for mi in range(g.batch):
        if kind == "gauss":
            v = a["std"] * randn(g.m, g.n)
        elif kind == "lowrank_noise":
            v = randn(g.m, a["k"]) @ randn(g.n, a["k"]).T + a["noise_std"] * randn(g.m, g.n)
        elif kind == "loguniform_gauss":
            v = scales[mi] * randn(g.m, g.n)
        elif kind == "student_t":
            # t_nu = Z / sqrt(chi2_nu / nu), chi2 of integer nu as a sum of nu squared normals
            nu = int(a["nu"])
            if nu != a["nu"]:
                raise ValueError("the device Student-t draw needs an integer nu")
            chi2 = sum(randn(g.m, g.n) ** 2 for _ in range(nu))
            v = a["scale"] * randn(g.m, g.n) / torch.sqrt(chi2 / nu)
        elif kind == "decaying_spectrum":
            n = g.n
            sig = 10.0 ** (-a["decades"] * torch.arange(n, device=device, dtype=torch.float64) / n)

            def haar():
                q, t = torch.linalg.qr(randn(n, n))
                return q * torch.sign(torch.diagonal(t))[None, :]
            U, V = haar(), haar()
            v = (U * sig[None, :]) @ V.T
        else:
            raise ValueError(f"unknown gradient recipe {kind!r}")
        out[mi] = _torch_store(v, dt)
    return out
