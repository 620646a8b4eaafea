"""Pins of the oracle's Adam (CPU)."""
import numpy as np
import torch

import oracle


def _seq(seed, shapes, steps, zero_frac=0.5):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(steps):
        gs = []
        for s in shapes:
            g = rng.standard_normal(s) * 1e-3
            g[..., rng.random(s[-1]) < zero_frac] = 0.0  # whole Gaussians (columns) without gradient
            gs.append(g)
        out.append(gs)
    return out


def test_matches_torch_adam():
    rng = np.random.default_rng(1)
    shapes = [(3, 50), (48, 50), (1, 50)]
    params = [rng.standard_normal(s) for s in shapes]
    lrs = [1.6e-4, 2.5e-3, 5e-2]
    seq = _seq(2, shapes, 12)
    p, m, v = oracle.adam(params, seq, lrs, 0.9, 0.999, 1e-15)
    tp = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in params]
    opt = torch.optim.Adam([{"params": [t], "lr": lr} for t, lr in zip(tp, lrs)], betas=(0.9, 0.999), eps=1e-15)
    for grads in seq:
        for t, g in zip(tp, grads):
            t.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    for a, b, lr in zip(p, tp, lrs):
        assert np.allclose(a, b.detach().numpy(), rtol=0, atol=1e-12 * lr * 12 + 1e-15)


def test_first_step_and_zero_gradient_decay():
    g = np.array([[3e-4, -2e-6, 0.0, 7.0]])
    p0 = np.array([[1.0, 2.0, 3.0, 4.0]])
    p, m, v = oracle.adam([p0], [[g]], [0.01], 0.9, 0.999, 1e-8)
    assert np.allclose(p[0], p0 - 0.01 * g / (np.abs(g) + 1e-8), rtol=0, atol=1e-15)
    # then k steps without gradient: the moments decay geometrically
    k = 5
    p2, m2, v2 = oracle.adam([p0], [[g]] + [[np.zeros_like(g)]] * k, [0.01], 0.9, 0.999, 1e-8)
    assert np.allclose(m2[0], 0.9 ** k * m[0], rtol=1e-15, atol=0)
    assert np.allclose(v2[0], 0.999 ** k * v[0], rtol=1e-15, atol=0)
    assert p2[0][0, 2] == 3.0  # never a gradient: never moves
