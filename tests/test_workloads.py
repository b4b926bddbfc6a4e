"""Seeded synthetic inputs: identical bits run to run, and the stated distributions."""
import numpy as np

import workloads as W


def test_seeded_bits_repeat():
    for wid in (1, 2, 3, 4, 5):
        wl = W.SMALL[wid]
        for gi in range(len(wl.groups)):
            a = W.make_grad(wl, gi, 2)
            b = W.make_grad(wl, gi, 2)
            assert a.tobytes() == b.tobytes()
            c = W.make_grad(wl, gi, 3)
            assert a.tobytes() != c.tobytes()        # fresh gradient every step
            X1, M1, Q1 = W.make_state(wl, gi)
            X2, M2, Q2 = W.make_state(wl, gi)
            assert X1.tobytes() == X2.tobytes() and Q1.tobytes() == Q2.tobytes()
            assert not M1.any()


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -3.0e-5, 65504.0], dtype=np.float32)
    b = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins; 1 + 1.5 * 2^-8 rounds up
    assert b[0] == 1.0 and b[1] == 1.0 and b[2] == 1.0078125 and b[3] == 1.0078125
    assert abs(b[4] - x[4]) <= abs(x[4]) * 2 ** -8


def test_distributions():
    wl = W.SMALL[1]
    X, M, Q = W.make_state(wl, 0)
    assert abs(X.std() - 0.02) < 0.002
    assert np.allclose(np.linalg.norm(Q[0].astype(np.float64), axis=0), 1.0, atol=1e-6)
    G = W.make_grad(wl, 0, 1)
    assert abs(G.std() - 1e-2) < 1e-3
    # low-rank + noise: rank-k signal dominates, noise floor at noise_std
    wl2 = W.SMALL[2]
    G2 = W.make_grad(wl2, 0, 1)[0].astype(np.float64)
    s = np.linalg.svd(G2, compute_uv=False)
    k = wl2.grad_args["k"]
    assert s[k - 1] > 100 * s[k]
    # per-matrix log-uniform scale within [lo, hi]
    wl3 = W.SMALL[3]
    G3 = W.to_f64(W.make_grad(wl3, 0, 1), "bf16")
    sd = G3.reshape(G3.shape[0], -1).std(axis=1)
    assert np.all(sd > 0.5e-5) and np.all(sd < 2e-2)
    # decaying spectrum: 10^(-6 i / n)
    wl5 = W.SMALL[5]
    G5 = W.make_grad(wl5, 0, 1)[0].astype(np.float64)
    s5 = np.linalg.svd(G5, compute_uv=False)
    n = G5.shape[0]
    assert abs(np.log10(s5[0] / s5[n // 2]) - 3.0) < 0.05


def test_device_generators_follow_the_recipes():
    """The benchmark's on-device draws (run here on torch's CPU device): the same distributions
    as the host generators, repeatable for a seed, fresh per step."""
    import torch
    dev = torch.device("cpu")
    wl = W.SMALL[1]
    X, M, Q = W.make_state_device(wl, 0, dev)
    assert X.dtype == torch.float32 and abs(float(X.std()) - 0.02) < 0.002 and not M.any()
    assert torch.allclose(torch.linalg.vector_norm(Q[0].double(), dim=0), torch.ones(wl.groups[0].rank,
                                                                                     dtype=torch.float64), atol=1e-6)
    G = W.make_grad_device(wl, 0, 1, dev)
    assert abs(float(G.std()) - 1e-2) < 1e-3
    assert torch.equal(G, W.make_grad_device(wl, 0, 1, dev)) and not torch.equal(G, W.make_grad_device(wl, 0, 2, dev))
    wl2 = W.SMALL[2]
    s = torch.linalg.svdvals(W.make_grad_device(wl2, 0, 1, dev)[0].double())
    k = wl2.grad_args["k"]
    assert s[k - 1] > 100 * s[k]
    wl3 = W.SMALL[3]
    G3 = W.make_grad_device(wl3, 0, 1, dev)
    assert G3.dtype == torch.bfloat16
    sd = G3.double().reshape(G3.shape[0], -1).std(dim=1)
    assert bool((sd > 0.5e-5).all()) and bool((sd < 2e-2).all())
    X3, _, _ = W.make_state_device(wl3, 0, dev)
    assert X3.dtype == torch.bfloat16
    # Student-t with nu = 3: symmetric, heavy tails (excess kurtosis of t_3 is infinite; the
    # sample's exceeds the Gaussian's 0 by far) and scale 1e-3 (median |t_3| = 0.765)
    wl4 = W.SMALL[4]
    G4 = W.make_grad_device(wl4, 0, 1, dev).double().flatten()
    med = float(G4.abs().median())
    assert 0.65e-3 < med < 0.88e-3
    z = (G4 - G4.mean()) / G4.std()
    assert float((z ** 4).mean()) - 3.0 > 3.0
    wl5 = W.SMALL[5]
    s5 = torch.linalg.svdvals(W.make_grad_device(wl5, 0, 1, dev)[0].double())
    n = s5.shape[0]
    assert abs(float(torch.log10(s5[0] / s5[n // 2])) - 3.0) < 0.05
