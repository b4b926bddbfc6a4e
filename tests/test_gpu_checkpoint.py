"""Checkpoint and resume: a stack stepped twice, saved (torch.save of DionStack.state_dict() and
the weights), restored into fresh tensors (torch.load with weights_only=True) and stepped twice
more ends bitwise where four uninterrupted steps end: X, M, Q and the flags.  The fp32
attention-like stack takes the sticky fp64 chain (its flags carry the mark across the save); the
bf16 stack takes the plain bf16 products."""
import pytest

import workloads as W
from tests.harness import to_torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wid", [2, 3])
def test_checkpoint_resume_is_bitwise(cuda, tmp_path, wid):
    import torch
    import rank_orthonormalized_optimizer_amd as dion
    wl = W.SMALL[wid]
    g = wl.groups[0]
    X0, _, Q0 = W.make_state(wl, 0)
    grads = [W.make_grad(wl, 0, t) for t in range(1, 5)]

    def stack():
        st = dion.DionStack(g.batch, g.m, g.n, rank=g.rank, mu=wl.mu, lr=wl.lr, eps=wl.eps, device=cuda)
        st.Q.copy_(to_torch(Q0, cuda))
        return st

    ref = stack()
    Xr = to_torch(X0, cuda)
    for G in grads:
        ref.step(Xr, to_torch(G, cuda))
    torch.cuda.synchronize()

    first = stack()
    Xa = to_torch(X0, cuda)
    for G in grads[:2]:
        first.step(Xa, to_torch(G, cuda))
    torch.cuda.synchronize()
    torch.save({"opt": first.state_dict(), "X": Xa.cpu()}, tmp_path / "ckpt.pt")
    del first, Xa

    ck = torch.load(tmp_path / "ckpt.pt", weights_only=True)
    resumed = stack()
    resumed.load_state_dict(ck["opt"])
    Xb = ck["X"].to(cuda)
    for G in grads[2:]:
        resumed.step(Xb, to_torch(G, cuda))
    torch.cuda.synchronize()
    assert torch.equal(Xb, Xr)
    assert torch.equal(resumed.M, ref.M)
    assert torch.equal(resumed.Q, ref.Q)
    assert torch.equal(resumed.flags, ref.flags)
    if wid == 2:
        assert bool((resumed.flags & dion.FLAG_F64).all())   # the fp64 mark survived the save


def test_load_state_dict_rejects_other_sizes(cuda):
    import rank_orthonormalized_optimizer_amd as dion
    a = dion.DionStack(2, 64, 48, rank=8, device=cuda)
    b = dion.DionStack(2, 64, 48, rank=16, device=cuda)
    with pytest.raises(ValueError):
        b.load_state_dict(a.state_dict())
