"""GPU parity of the element-wise optimizers (AdamW, Lion) against the fp64 oracle.

Teacher-forced like the Dion step: every step starts the oracle from the state the
GPU stored.  Inputs are seeded and synthetic (weights ~ N(0, 0.02^2), gradients
~ N(0, 1e-4), the scales of the Dion workloads' 1-D companions), stored as fp32 or
bf16.  Sizes cover the empty array, tails of one to three elements after the
four-wide groups, several grid strides, and a 2^22-element array.

The oracle takes the hyper-parameters as the fp32 values the C ABI receives.
Bar: relative Frobenius error <= 1e-4 on the parameter for fp32 storage and
<= 2e-2 for bf16 (one rounding to bf16 per step), <= 1e-5 on the fp32 moments.
Lion's direction is a sign, decided in fp32 on the GPU: it must agree with the
oracle's everywhere the blended momentum is not at fp32 rounding level.
"""
import numpy as np
import pytest

from oracle.elementwise_oracle import adamw_step, lion_step
from tests.harness import rel, to_numpy, to_torch

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 3, 4, 7, 1027, 65536 + 5, 1 << 22]
DTYPES = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16")]


def _store(x, dt):
    x = np.asarray(x, np.float64)
    if dt == "f32":
        return x.astype(np.float32)
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)   # round to nearest even
    return u


def _up(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _rel(a, b):
    return rel(_up(a), b) if np.linalg.norm(b) > 0 else float(np.linalg.norm(_up(a) - b))


@pytest.mark.parametrize("pdt,gdt", DTYPES)
@pytest.mark.parametrize("n", SIZES)
def test_adamw_parity(cuda, n, pdt, gdt):
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([11, n, len(pdt), len(gdt)])))
    p = to_torch(_store(0.02 * rng.standard_normal(n), pdt), cuda)
    m = torch.zeros(n, dtype=torch.float32, device=cuda)
    v = torch.zeros(n, dtype=torch.float32, device=cuda)
    # the hyper-parameters as the fp32 values the library receives (its inputs, exactly upcast)
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (1e-3, 0.9, 0.999, 1e-8, 0.1))
    tol = 1e-4 if pdt == "f32" else 2e-2
    for t in range(1, 4):
        g_np = _store(1e-2 * rng.standard_normal(n), gdt)
        pre = (to_numpy(p), to_numpy(m), to_numpy(v))
        print(f"[elementwise] adamw n={n} p={pdt} g={gdt} step {t}", flush=True)
        dion.adamw_step_(p, to_torch(g_np, cuda), m, v, t, lr, b1, b2, eps, wd)
        torch.cuda.synchronize()
        th, mm, vv = adamw_step(_up(pre[0]), _up(g_np), _up(pre[1]), _up(pre[2]), t, lr, b1, b2, eps, wd)
        if n == 0:
            continue
        assert _rel(to_numpy(p), th) <= tol
        assert _rel(to_numpy(m), mm) <= 1e-5
        assert _rel(to_numpy(v), vv) <= 1e-5


@pytest.mark.parametrize("pdt,gdt", DTYPES)
@pytest.mark.parametrize("n", SIZES)
def test_lion_parity(cuda, n, pdt, gdt):
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([12, n, len(pdt), len(gdt)])))
    p = to_torch(_store(0.02 * rng.standard_normal(n), pdt), cuda)
    m = torch.zeros(n, dtype=torch.float32, device=cuda)
    lr, b1, b2, wd = (float(np.float32(x)) for x in (3e-4, 0.9, 0.99, 0.1))
    tol = 1e-4 if pdt == "f32" else 2e-2
    for t in range(1, 4):
        g_np = _store(1e-2 * rng.standard_normal(n), gdt)
        if n:
            g_np[:: max(1, n // 7)] = 0   # exact zeros: sign 0 on the first step
        pre = (to_numpy(p), to_numpy(m))
        print(f"[elementwise] lion n={n} p={pdt} g={gdt} step {t}", flush=True)
        dion.lion_step_(p, to_torch(g_np, cuda), m, lr, b1, b2, wd)
        torch.cuda.synchronize()
        th, mm = lion_step(_up(pre[0]), _up(g_np), _up(pre[1]), lr, b1, b2, wd)
        if n == 0:
            continue
        assert _rel(to_numpy(p), th) <= tol
        assert _rel(to_numpy(m), mm) <= 1e-5
        if pdt == "f32":   # the direction, wherever the blend is clear of fp32 rounding
            c = b1 * _up(pre[1]) + (1 - b1) * _up(g_np)
            scale = np.abs(b1 * _up(pre[1])) + np.abs((1 - b1) * _up(g_np))
            clear = np.abs(c) > 1e-6 * scale
            move = _up(pre[0]) * (1 - lr * wd) - _up(to_numpy(p))
            assert np.all(np.sign(move[clear & (np.abs(move) > lr / 2)]) == np.sign(c[clear & (np.abs(move) > lr / 2)]))
            assert np.all(np.abs(np.abs(move[clear]) - lr) < 1e-3 * lr + 1e-7)
