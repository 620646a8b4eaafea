"""The HIP path on the golden scene against the oracle's stored results
(tests/golden/tiny_two_views.json, written by tests/golden/make_golden.py from the oracle):
end to end, projection -> bins -> fused forward, L1 gradient and backward, for both views.
Needs an MI355X."""
import json
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


@pytest.fixture(scope="module")
def run():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    from differentiable_raster_amd import pipeline
    sc = make_golden.golden_scene()
    r = pipeline.Renderer(sc, sc.settings())
    print("[golden] fused iteration and separate forward, 2 views of 48x32", flush=True)
    r.iteration(mode="fused", image=True)
    torch.cuda.synchronize()
    image = r.images_host()[0]
    grads = [r.grads_host(v) for v in range(r.V)]
    r.forward()  # transmittance and n_contrib (the fused call keeps them in registers)
    torch.cuda.synchronize()
    _, T, nc = r.images_host()
    return dict(stored=json.load(open(make_golden.FIXTURE)), r=r, image=image, T=T, nc=nc, grads=grads)


def test_projection_and_bins(run):
    r, stored = run["r"], run["stored"]
    for v, o in enumerate(stored["views"]):
        g = r.projected_host(v)
        assert g["vis_ids"].tolist() == o["vis_ids"]
        assert (g["rect"].tolist(), g["n_tiles"].tolist()) == (o["rect"], o["n_tiles"])
        # float32 against float64: a few ulp of each output, with the conic scaled by its largest
        # entry (it is the inverse of the dilated covariance)
        m, con = np.asarray(o["mean2d"]), np.asarray(o["conic"])
        assert (np.abs(g["mean2d"] - m) <= 1e-5 * np.abs(m) + 1e-4).all()
        scale = np.abs(con).max(axis=1, keepdims=True)
        assert (np.abs(g["conic_opacity"][:, :3] - con) <= 1e-5 * scale).all()
        assert np.allclose(g["conic_opacity"][:, 3], o["opacity"], rtol=1e-6, atol=1e-7)
        assert np.allclose(g["color"], o["color"], rtol=1e-5, atol=1e-6)
        assert np.allclose(g["depth"], o["depth"], rtol=1e-6, atol=0.0)
        b = r.bins_host(v)
        assert b["ranges"].tolist() == o["ranges"] and b["vals"].tolist() == o["vals"]


def test_pixels(run):
    stored = run["stored"]
    for v, o in enumerate(stored["views"]):
        assert o["flagged_pixels"] == 0
        img = run["image"][v]
        # the image sums: every pixel's float32 error bound, summed
        s = img.astype(np.float64).sum(axis=(1, 2))
        tol = 1e-5 * np.abs(o["image_sum"]) + np.asarray(o["image_sum_err"]) + 1e-7 * img[0].size
        assert (np.abs(s - o["image_sum"]) <= tol).all(), (s, o["image_sum"])
        for p in o["pixels"]:
            x, y = p["x"], p["y"]
            c = img[:, y, x].astype(np.float64)
            assert (np.abs(c - p["C"]) <= 1e-5 * np.abs(p["C"]) + 1e-7 + np.asarray(p["err_C"])).all(), p
            assert abs(float(run["T"][v, y, x]) - p["T"]) <= (1e-5 + p["err_T"]) * p["T"] + 1e-7, p
            assert int(run["nc"][v, y, x]) == p["n_contrib"], p


def test_gradients_2d(run):
    stored = run["stored"]
    for v, o in enumerate(stored["views"]):
        g = run["grads"][v]
        gpu = np.concatenate([g["d_mean2d"], g["d_conic"], g["d_opacity"][:, None], g["d_color"]], axis=1)
        ref = np.concatenate([np.asarray(o["d_mean2d"]), np.asarray(o["d_conic"]),
                              np.asarray(o["d_opacity"])[:, None], np.asarray(o["d_color"])], axis=1)
        use = ~np.asarray(o["slot_flag"])
        # the survey's gradient tolerance plus the oracle's float32 bound of each component
        tol = 1e-3 * np.abs(ref) + 1e-6 + np.asarray(o["grad_bound"])
        bad = np.abs(gpu.astype(np.float64) - ref) > tol
        assert not bad[use].any(), np.argwhere(bad & use[:, None])[:5]
