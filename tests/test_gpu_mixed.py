"""GPU check of the mixed optimizer: Dion for the 2-D parameters, AdamW or Lion for the rest.

rivista.ai, the paragraph beginning "Tecnicamente": Dion takes the 2-D weights and
leaves biases and other tensors to an element-wise optimizer.  ``MixedDion`` groups
the 2-D parameters by shape into stacks and steps the rest element-wise; this test
drives it for two steps over parameters of several shapes (two matrix shapes, one
of them a stack of three; a bias; a ragged 1-D tensor; a 3-D tensor) and checks
every parameter against the oracles, teacher-forced from the state the GPU holds
before each step.  Inputs are seeded and synthetic: weights ~ N(0, 0.02^2), gradients
~ N(0, 1e-4).  Bars as in the other parity tests: relative Frobenius error <= 1e-4 on
X', M' and P Q'^T for the Dion parameters, <= 1e-4 on the element-wise parameters and
<= 1e-5 on their fp32 moments.
"""
import numpy as np
import pytest

from oracle.dion_oracle import dion_step
from oracle.elementwise_oracle import adamw_step, lion_step
from tests.harness import rel, to_numpy

pytestmark = pytest.mark.gpu

SHAPES = [(64, 96), (64, 96), (96,), (64, 96), (128, 64), (7,), (2, 3, 5)]


def _f32(x):
    return float(np.float32(x))


@pytest.mark.parametrize("other", ["adamw", "lion"])
def test_mixed_optimizer_steps(cuda, other):
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([21, len(other)])))
    params = [torch.from_numpy((0.02 * rng.standard_normal(s)).astype(np.float32)).to(cuda) for s in SHAPES]
    lr, mu, other_lr, betas, eps, wd = 0.01, 0.95, 1e-3, (0.9, 0.99), 1e-8, 0.1
    opt = dion.MixedDion(params, lr=lr, mu=mu, rank_fraction=0.25, other=other, other_lr=other_lr, betas=betas,
                         eps=eps, weight_decay=wd)
    assert [idx for idx, _ in opt.groups] == [[0, 1, 3], [4]]
    assert opt.rest == [2, 5, 6]
    hb1, hb2, heps, hwd, hlr = _f32(betas[0]), _f32(betas[1]), _f32(eps), _f32(wd), _f32(other_lr)
    for t in (1, 2):
        grads = [torch.from_numpy((1e-2 * rng.standard_normal(s)).astype(np.float32)).to(cuda) for s in SHAPES]
        pre_p = [to_numpy(p).astype(np.float64) for p in params]
        pre_dion = [(to_numpy(st.M).astype(np.float64), to_numpy(st.Q).astype(np.float64)) for _, st in opt.groups]
        pre_ew = {i: tuple(None if s is None else to_numpy(s).astype(np.float64) for s in opt.state[i])
                  for i in opt.rest}
        print(f"[mixed] {other} step {t}", flush=True)
        opt.step(grads)
        torch.cuda.synchronize()
        g = [to_numpy(x).astype(np.float64) for x in grads]
        for (idx, st), (M0, Q0) in zip(opt.groups, pre_dion):
            P = to_numpy(st.P).astype(np.float64)
            Mg, Qg = to_numpy(st.M).astype(np.float64), to_numpy(st.Q).astype(np.float64)
            for k, i in enumerate(idx):
                o = dion_step(pre_p[i], g[i], M0[k], Q0[k], mu, _f32(lr), 1e-8)
                assert rel(to_numpy(params[i]).astype(np.float64), o["X"]) <= 1e-4, (t, i)
                assert rel(Mg[k], o["M"]) <= 1e-4, (t, i)
                assert rel(P[k] @ Qg[k].T, o["P"] @ o["Q"].T) <= 1e-4, (t, i)
        for i in opt.rest:
            got = to_numpy(params[i]).astype(np.float64).ravel()
            m0 = pre_ew[i][0]
            if other == "adamw":
                th, mm, vv = adamw_step(pre_p[i].ravel(), g[i].ravel(), m0, pre_ew[i][1], t, hlr, hb1, hb2, heps, hwd)
                assert rel(to_numpy(opt.state[i][1]).astype(np.float64), vv) <= 1e-5, (t, i)
            else:
                th, mm = lion_step(pre_p[i].ravel(), g[i].ravel(), m0, hlr, hb1, hb2, hwd)
            assert rel(got, th) <= 1e-4, (t, i)
            assert rel(to_numpy(opt.state[i][0]).astype(np.float64), mm) <= 1e-5, (t, i)
            assert tuple(params[i].shape) == SHAPES[i]


def test_mixed_optimizer_bf16(cuda):
    """bf16 weights: the 2-D ones go to Dion with bf16 X (fp32 M and Q), the rest to AdamW with a
    bf16 parameter; one step against the oracles at the bf16 bar (2e-2 on the parameters)."""
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    from tests.test_gpu_elementwise import _store, _up
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([22])))
    shapes = [(64, 96), (64, 96), (33,)]
    host = [_store(0.02 * rng.standard_normal(s), "bf16") for s in shapes]
    params = [torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(cuda) for h in host]
    opt = dion.MixedDion(params, lr=0.01, mu=0.95, other="adamw", other_lr=1e-3, betas=(0.9, 0.999),
                         weight_decay=0.0)
    gh = [_store(1e-2 * rng.standard_normal(s), "bf16") for s in shapes]
    grads = [torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(cuda) for h in gh]
    (idx, st), = opt.groups
    M0, Q0 = to_numpy(st.M).astype(np.float64), to_numpy(st.Q).astype(np.float64)
    print("[mixed] bf16 step", flush=True)
    opt.step(grads)
    torch.cuda.synchronize()
    for k, i in enumerate(idx):
        o = dion_step(_up(host[i]), _up(gh[i]), M0[k], Q0[k], 0.95, _f32(0.01), 1e-8)
        assert rel(_up(to_numpy(params[i])), o["X"]) <= 2e-2, i
    th, _, _ = adamw_step(_up(host[2]), _up(gh[2]), np.zeros(33), np.zeros(33), 1, _f32(1e-3), _f32(0.9),
                          _f32(0.999), _f32(1e-8), 0.0)
    assert rel(_up(to_numpy(params[2])), th) <= 2e-2
