"""Adam on the GPU (gs_adam_step / gs_adam_flush): dense against the oracle's float64 Adam, and the
deferred update against the dense one bit for bit (needs an MI355X)."""
import numpy as np
import pytest


pytestmark = pytest.mark.gpu

ROWS = [3, 3, 4, 1, 48]  # means, log-scales, quaternions, opacity logit, SH degree 3
LRS = [1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3]


@pytest.fixture(scope="module")
def env(oracle_mod):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    from differentiable_raster_amd import adam, gsmi
    gsmi.load()
    return oracle_mod, torch, adam


def _grad_seq(n, steps, seed):
    """Per step and group [rows][n] float32 gradients; a random half of the Gaussians has none."""
    rng = np.random.default_rng(seed)
    seq = []
    for _ in range(steps):
        zero = rng.random(n) < 0.5
        gs = []
        for r in ROWS:
            g = (rng.standard_normal((r, n)) * 1e-3).astype(np.float32)
            g[:, zero] = 0.0
            gs.append(g)
        seq.append((gs, np.nonzero(~zero)[0].astype(np.int32)))
    return seq


def _state(torch, adam, params, deferred):
    p = [torch.from_numpy(x.reshape(-1).copy()).cuda() for x in params]
    g = [torch.zeros_like(t) for t in p]
    st = adam.AdamState(params[0].shape[1], [(pt, gt, r, lr) for pt, gt, r, lr in zip(p, g, ROWS, LRS)],
                        deferred=deferred)
    return st, p, g


def _run(torch, adam, params, seq, mode):
    st, p, g = _state(torch, adam, params, deferred=mode != "dense")
    for gs, ids in seq:
        for dst, src in zip(g, gs):
            dst.copy_(torch.from_numpy(src.reshape(-1)))
        if mode == "active":
            # the Gaussians with a gradient, plus some without: listing them too changes nothing
            extra = np.arange(0, params[0].shape[1], 7, dtype=np.int32)
            st.step(torch.from_numpy(np.union1d(ids, extra).astype(np.int32)).cuda())
        elif mode == "seen":
            # flags on the Gaussians with a gradient and some without; the gradient rows of the
            # unflagged ones hold NaN, which the step must not read
            n = params[0].shape[1]
            flag = np.zeros(n, np.uint8)
            flag[ids] = 1
            flag[::7] = 1
            for dst, src in zip(g, gs):
                h = src.copy()
                h[:, flag == 0] = np.nan
                dst.copy_(torch.from_numpy(h.reshape(-1)))
            st.step(seen=torch.from_numpy(flag).cuda())
        else:
            st.step()
    st.flush()
    torch.cuda.synchronize()
    host = lambda ts: [t.cpu().numpy().reshape(r, -1) for t, r in zip(ts, ROWS)]
    return host(p), host(st.m), host(st.v), (st.last_step.cpu().numpy() if st.last_step is not None else None)


@pytest.mark.parametrize("n", [1000, 4097])
def test_dense_adam_matches_the_oracle(env, n):
    oracle, torch, adam = env
    rng = np.random.default_rng(n)
    params = [rng.standard_normal((r, n)).astype(np.float32) for r in ROWS]
    seq = _grad_seq(n, 15, seed=n + 1)
    p, m, v, _ = _run(torch, adam, params, seq, "dense")
    # the library takes its constants as float32 values (1 - 0.999f differs from 1 - 0.999 by 1.3e-5)
    f32 = lambda x: float(np.float32(x))
    rp, rm, rv = oracle.adam(params, [gs for gs, _ in seq], [f32(x) for x in LRS], f32(0.9), f32(0.999), f32(1e-15))
    for k, lr in enumerate(LRS):
        tol = 2e-6 * np.abs(rp[k]) + 1e-4 * lr * len(seq)
        assert (np.abs(p[k] - rp[k]) <= tol).all(), k
        # moments: float32 sums of terms of both signs, so the error scales with the moments' size
        assert np.abs(m[k] - rm[k]).max() <= 1e-5 * np.abs(rm[k]).max(), k
        assert np.abs(v[k] - rv[k]).max() <= 1e-5 * np.abs(rv[k]).max(), k


@pytest.mark.parametrize("mode", ["deferred", "active", "seen"])
def test_deferred_adam_equals_dense_bit_for_bit(env, mode):
    oracle, torch, adam = env
    n = 3000
    rng = np.random.default_rng(7)
    params = [rng.standard_normal((r, n)).astype(np.float32) for r in ROWS]
    seq = _grad_seq(n, 12, seed=8)
    print(f"[adam] {mode}: n={n}, {len(seq)} steps", flush=True)
    dense = _run(torch, adam, params, seq, "dense")
    lazy = _run(torch, adam, params, seq, mode)
    for a, b in zip(dense[:3], lazy[:3]):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    assert (lazy[3][:n] == len(seq)).all()
