"""Sparse 2D gradient encoder/decoder (gs_grad_encode / gs_grad_decode) vs the oracle, through the
C ABI (needs an MI355X).  Integer outputs and records bit for bit; the decoder's float32 adds bit
for bit against the same float32 additions in NumPy."""
import numpy as np
import pytest

from differentiable_raster_amd import scenes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env(oracle_mod):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    from differentiable_raster_amd import gsmi, sparse
    gsmi.load()
    return oracle_mod, torch, gsmi, sparse


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def _upload_grads(torch, gsmi, V, cap, per_view):
    """Slot-indexed [V][cap][...] gradient arrays; slots past vis_count hold garbage."""
    rng = np.random.default_rng(99)
    full = rng.standard_normal((V, cap, 9)).astype(np.float32)  # garbage beyond the visible slots
    for v, R in enumerate(per_view):
        full[v, :R.shape[0]] = R
    t = [torch.from_numpy(np.ascontiguousarray(full[:, :, a:b])).reshape(-1).cuda()
         for a, b in ((0, 2), (2, 5), (5, 6), (6, 9))]
    return t, gsmi.gs_grads2d(t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), t[3].data_ptr())


@pytest.mark.parametrize("case", [(3, 1000, [1000, 517, 0], 0.3), (1, 257, [257], 0.0), (2, 64, [1, 64], 1.0)])
def test_encode_decode_match_the_oracle(env, case):
    oracle, torch, gsmi, sparse = env
    V, cap, counts, density = case
    n_owner = 3 * cap + 5
    print(f"[sparse] V={V} capacity={cap} vis_count={counts} density={density}", flush=True)
    rng = np.random.default_rng(cap + V)
    vis_ids = np.full((V, cap), -1, np.int32)
    per_view = []
    for v, n in enumerate(counts):
        vis_ids[v, :n] = np.sort(rng.choice(n_owner, size=n, replace=False))
        R = rng.standard_normal((n, 9)).astype(np.float32)
        R[rng.random(n) >= density] = 0.0
        if n > 8:
            R[3] = -0.0
            R[4, :] = 0.0
            R[4, 7] = np.nan
            R[5, :] = 0.0
            R[5, 0] = -1e-38
        per_view.append(R)
    t, grads = _upload_grads(torch, gsmi, V, cap, per_view)
    vis_count_d = torch.tensor(counts, dtype=torch.int32, device="cuda")
    vis_ids_d = torch.from_numpy(vis_ids.reshape(-1)).cuda()
    codec = sparse.GradCodec(V, cap, n_owner)
    codec.encode(vis_count_d, vis_ids_d, grads)
    torch.cuda.synchronize()
    got = codec.encoded_host()
    ref = oracle.grad_encode(counts, vis_ids, per_view)
    assert list(got["view_offset"]) == list(ref["view_offset"])
    assert np.array_equal(got["keys"], ref["keys"])
    assert np.array_equal(_bits(got["records"]), _bits(ref["records"]))
    # decode into owner arrays that already hold values: one float32 add per component
    init = rng.standard_normal((V, n_owner, 9)).astype(np.float32)
    for dst, (a, b) in zip((codec.o_mean2d, codec.o_conic, codec.o_opacity, codec.o_color),
                           ((0, 2), (2, 5), (5, 6), (6, 9))):
        dst.copy_(torch.from_numpy(np.ascontiguousarray(init[:, :, a:b])).reshape(-1))
    codec.decode()
    torch.cuda.synchronize()
    want = oracle.grad_decode(ref["view_offset"], ref["keys"], ref["records"], init, dtype=np.float32)
    assert np.array_equal(_bits(codec.owner_host()), _bits(want))
    kept = int(ref["view_offset"][-1])
    print(f"[sparse] kept {kept} of {sum(counts)} records", flush=True)


def test_round_trip_of_a_fused_backward_equals_the_dense_scatter(env):
    oracle, torch, gsmi, sparse = env
    from differentiable_raster_amd import pipeline
    sc = scenes.random_scene(20000, 320, 240, seed=11, views=3, log_scale_mean=-3.0)
    r = pipeline.Renderer(sc, sc.settings())
    r.iteration(mode="fused")
    codec = sparse.GradCodec(r.V, r.capacity, r.n)
    codec.encode(r.vis_count, r.vis_ids, r.grads)
    codec.decode()
    torch.cuda.synchronize()
    own = codec.owner_host()
    dense = np.zeros_like(own)
    total = 0
    for v in range(r.V):
        g = r.grads_host(v)
        ids = r.projected_host(v)["vis_ids"]
        dense[v, ids] = np.concatenate([g["d_mean2d"], g["d_conic"], g["d_opacity"][:, None], g["d_color"]], axis=1)
        total += ids.size
    assert np.array_equal(own, dense)
    kept = int(codec.view_offset[-1].item())
    print(f"[sparse] fused backward: {kept} of {total} records non-zero ({100.0 * (1 - kept / total):.1f} % dropped)",
          flush=True)
