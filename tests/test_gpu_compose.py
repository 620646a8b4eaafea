"""Composition of partial renders (gs_compose) on the GPU: against the oracle's composition of the
same partials, and against rendering the union when the subsets are depth-separated (needs an
MI355X)."""
import numpy as np
import pytest

from helpers import depth_layered_scene, subset

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env(oracle_mod):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    from differentiable_raster_amd import gsmi, pipeline
    gsmi.load()
    return oracle_mod, torch, gsmi, pipeline


def _render(pipeline, torch, scene, settings):
    r = pipeline.Renderer(scene, settings)
    r.project()
    r.bin()
    r.forward()
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("layers,views", [(((2.0, 3.0), (4.0, 5.0), (6.5, 8.0)), 2), (((2.0, 3.5), (5.0, 9.0)), 1)])
def test_depth_separated_partials_compose_to_the_union(env, layers, views):
    oracle, torch, gsmi, pipeline = env
    sc, idx = depth_layered_scene(400, 150, 100, seed=21, layers=layers, views=views)
    print(f"[compose] {sc.name}: {len(layers)} layers, {views} views", flush=True)
    bg = (0.25, 0.5, 0.75)
    full = _render(pipeline, torch, sc, sc.settings(t_min=0.0, bg=bg))
    parts = [_render(pipeline, torch, subset(sc, i), sc.settings(t_min=0.0)) for i in idx]
    V, H, W = full.V, full.H, full.W
    img = torch.empty(V * 3 * H * W, dtype=torch.float32, device="cuda")
    T = torch.empty(V * H * W, dtype=torch.float32, device="cuda")
    gsmi.gs_compose(V, W, H, [p.image for p in parts], [p.t_final for p in parts], bg, img, T)
    torch.cuda.synchronize()
    img_h, T_h = img.view(V, 3, H, W).cpu().numpy(), T.view(V, H, W).cpu().numpy()
    # the composition of these partials, by the oracle (float64)
    ref_img, ref_T = oracle.compose([p.images_host()[0] for p in parts], [p.images_host()[1] for p in parts],
                                    [float(np.float32(x)) for x in bg])
    assert np.abs(img_h - ref_img).max() <= 1e-6 * max(1.0, np.abs(ref_img).max())
    assert np.abs(T_h - ref_T).max() <= 1e-6
    # against compositing the union in one pass (float32 both ways: different rounding order)
    f_img, f_T, _ = full.images_host()
    assert f_T.min() < 0.9
    err = np.abs(img_h - f_img).max()
    print(f"[compose] max |composed - union| = {err:.3g}", flush=True)
    assert err <= 1e-5 * max(1.0, np.abs(f_img).max())
    assert np.abs(T_h - f_T).max() <= 1e-5


def test_single_partial_and_in_place_output(env):
    oracle, torch, gsmi, pipeline = env
    rng = np.random.default_rng(5)
    V, H, W = 2, 37, 53
    c = torch.from_numpy(rng.random(V * 3 * H * W, dtype=np.float32)).cuda()
    t = torch.from_numpy(rng.random(V * H * W, dtype=np.float32)).cuda()
    c0, t0 = c.clone(), t.clone()
    bg = (0.5, 0.0, 1.0)
    gsmi.gs_compose(V, W, H, [c], [t], bg, c, t)  # in place
    torch.cuda.synchronize()
    want = c0.view(V, 3, H, W) + t0.view(V, 1, H, W) * torch.tensor(bg, device="cuda").view(1, 3, 1, 1)
    assert torch.allclose(c.view(V, 3, H, W), want, rtol=0, atol=1e-6)
    assert torch.equal(t, t0)
