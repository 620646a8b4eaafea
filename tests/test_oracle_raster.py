"""Pins of the oracle's forward compositing: closed forms, telescoping identities and a
brute-force (no tiles, no binning) renderer."""
import math

import numpy as np
import pytest

from differentiable_raster_amd import scenes
from helpers import logit, pinhole, scene_from


def widen(x):
    return float(np.float32(x))


def render(oracle_mod, sc, st, view=0):
    return oracle_mod.iteration(sc, st, views=[view], backward=False)[0]


def test_single_gaussian_profile(oracle_mod):
    """One isotropic Gaussian on the optical axis, centred on pixel (32, 32):
    C(p) = c min(alpha_max, o exp(-r^2 / 2 s'^2)) where that reaches alpha_min, else 0,
    with s'^2 = (f s / z)^2 + eps; T = 1 - alpha."""
    f, z, ls, o = 80.0, 3.0, -2.4, 0.8
    cam = pinhole(64, 64, f=f, cx=32.5, cy=32.5)
    col = [0.9, 0.5, 0.25]
    sc = scene_from([[0, 0, z]], [[ls] * 3], [[0.3, 0.1, -0.5, 0.2]], [logit(o)], [col], [cam])
    st = sc.settings()
    r = render(oracle_mod, sc, st)
    ys, xs = np.mgrid[0:64, 0:64]
    r2 = (xs + 0.5 - 32.5) ** 2 + (ys + 0.5 - 32.5) ** 2
    var = (f * math.exp(widen(ls)) / z) ** 2 + widen(0.3)
    o32 = 1 / (1 + math.exp(-widen(logit(o))))
    v = o32 * np.exp(-r2 / (2 * var))
    alpha = np.minimum(widen(0.99), v)
    alpha = np.where(alpha >= widen(1 / 255), alpha, 0.0)
    for ch in range(3):
        np.testing.assert_allclose(r["fwd"]["image"][ch], widen(col[ch]) * alpha, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["fwd"]["T_final"], 1 - alpha, rtol=1e-12, atol=1e-15)
    assert (r["fwd"]["n_contrib"] == (alpha > 0)).all()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_telescoping_identities(oracle_mod, seed):
    """With every colour 1: background 0 gives C = 1 - T_final; background 1 gives C = 1."""
    sc = scenes.random_scene(600, 80, 64, seed=seed, log_scale_mean=-2.8, opacity_std=1.5)
    sc.sh[0:3] = 1.0
    st0 = sc.settings()
    r0 = render(oracle_mod, sc, st0)
    for ch in range(3):
        np.testing.assert_allclose(r0["fwd"]["image"][ch], 1 - r0["fwd"]["T_final"], rtol=0, atol=1e-13)
    st1 = sc.settings(bg=(1.0, 1.0, 1.0))
    r1 = render(oracle_mod, sc, st1)
    np.testing.assert_allclose(r1["fwd"]["image"], 1.0, rtol=0, atol=1e-13)
    assert r0["fwd"]["n_blended"] > 10000


def test_two_gaussians_and_termination(oracle_mod):
    """Stacked Gaussians on the axis, seen at the pixel they are centred on (G = 1 there):
    C = sum_k alpha_k T_k c_k with T_k = prod_{i<k} (1 - alpha_i); the walk stops before the
    blend that would take T below t_min, and that entry is not blended."""
    cam = pinhole(32, 32, f=40.0, cx=16.5, cy=16.5)
    o = [0.6, 0.7]
    cols = [[0.9, 0.1, 0.2], [0.3, 0.8, 0.4]]
    sc = scene_from([[0, 0, 2.0], [0, 0, 3.0]], [[-2.5] * 3, [-2.2] * 3], [[1, 0, 0, 0]] * 2,
                    [logit(o[0]), logit(o[1])], cols, [cam])
    r = render(oracle_mod, sc, sc.settings())
    a1, a2 = [1 / (1 + math.exp(-widen(logit(v)))) for v in o]
    c1, c2 = np.float32(cols[0]).astype(float), np.float32(cols[1]).astype(float)
    np.testing.assert_allclose(r["fwd"]["image"][:, 16, 16], a1 * c1 + (1 - a1) * a2 * c2, rtol=1e-12)
    np.testing.assert_allclose(r["fwd"]["T_final"][16, 16], (1 - a1) * (1 - a2), rtol=1e-12)
    assert r["fwd"]["n_contrib"][16, 16] == 2

    # five opaque Gaussians (alpha 0.95 at the centre): T = 0.05, 0.0025, 1.25e-4, then the
    # fourth would take T to 6.25e-6 < 1e-4: three blends, n_contrib 3
    k = 5
    sc = scene_from([[0, 0, 2.0 + i] for i in range(k)], [[-2.5] * 3] * k, [[1, 0, 0, 0]] * k,
                    [logit(0.95)] * k, [[0.1 * (i + 1)] * 3 for i in range(k)], [cam])
    r = render(oracle_mod, sc, sc.settings())
    a = 1 / (1 + math.exp(-widen(logit(0.95))))
    Ts = [1.0, 1 - a, (1 - a) ** 2]
    expect = sum(a * Ts[i] * widen(0.1 * (i + 1)) for i in range(3))
    np.testing.assert_allclose(r["fwd"]["image"][0, 16, 16], expect, rtol=1e-12)
    np.testing.assert_allclose(r["fwd"]["T_final"][16, 16], (1 - a) ** 3, rtol=1e-12)
    assert r["fwd"]["n_contrib"][16, 16] == 3


def test_alpha_clamp(oracle_mod):
    """An opacity above alpha_max at the centre is clamped to alpha_max."""
    cam = pinhole(32, 32, f=40.0, cx=16.5, cy=16.5)
    sc = scene_from([[0, 0, 2.0]], [[-2.0] * 3], [[1, 0, 0, 0]], [logit(0.999)], [[1, 1, 1]], [cam])
    r = render(oracle_mod, sc, sc.settings())
    np.testing.assert_allclose(r["fwd"]["T_final"][16, 16], 1 - widen(0.99), rtol=1e-15)


def numpy_bruteforce(rec, width, height, st):
    """Every visible Gaussian composited at every pixel, in (depth, slot) order: no tiles."""
    order = np.lexsort((np.arange(rec["vis_count"]), rec["depth"].astype(np.float32)))
    ys, xs = np.mgrid[0:height, 0:width]
    px, py = xs + 0.5, ys + 0.5
    C = np.zeros((3, height, width))
    T = np.ones((height, width))
    active = np.ones((height, width), bool)
    amin, amax, tmin = widen(st.alpha_min), widen(st.alpha_max), widen(st.t_min)
    for s in order:
        A, B, Cc = rec["conic"][s]
        dx, dy = px - rec["mean2d"][s, 0], py - rec["mean2d"][s, 1]
        alpha = np.minimum(amax, rec["opacity"][s] * np.exp(-0.5 * (A * dx * dx + 2 * B * dx * dy + Cc * dy * dy)))
        blend = active & (alpha >= amin)
        Tn = T * (1 - alpha)
        stop = blend & (Tn < tmin)
        active &= ~stop
        blend &= ~stop
        for ch in range(3):
            C[ch] += np.where(blend, alpha * T * rec["color"][s, ch], 0.0)
        T = np.where(blend, Tn, T)
    for ch in range(3):
        C[ch] += T * widen(st.bg[ch])
    return C, T


@pytest.mark.parametrize("seed,views", [(21, 1), (22, 2), (23, 2)])
def test_tiled_equals_bruteforce(oracle_mod, seed, views):
    sc = scenes.random_scene(500, 72, 56, seed=seed, views=views, log_scale_mean=-2.6, log_scale_std=0.7,
                             opacity_std=1.5, sh_degree=1)
    st = sc.settings()
    for v in range(views):
        r = render(oracle_mod, sc, st, view=v)
        C, T = numpy_bruteforce(r["rec"], sc.cameras[v].width, sc.cameras[v].height, st)
        np.testing.assert_allclose(r["fwd"]["image"], C, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r["fwd"]["T_final"], T, rtol=1e-12, atol=1e-14)
        assert r["fwd"]["n_blended"] > 5000


def test_tiled_equals_c_bruteforce_bitwise(oracle_mod):
    """The C brute force walks all slots in (depth, slot) order; tiling only removes pairs
    below alpha_min, so image and T agree bit for bit."""
    sc = scenes.make_scene(1)
    st = sc.settings()
    r = render(oracle_mod, sc, st)
    rec = r["rec"]
    order = np.lexsort((np.arange(rec["vis_count"]), rec["depth"].astype(np.float32))).astype(np.int32)
    b = oracle_mod.raster_bruteforce(128, 128, order, rec, st)
    assert np.array_equal(b["image"], r["fwd"]["image"])
    assert np.array_equal(b["T_final"], r["fwd"]["T_final"])


def test_anisotropic_profile_with_library_inverse(oracle_mod):
    """A Gaussian rotated 45 degrees about the optical axis has an off-diagonal 2D covariance:
    (f/z)^2 Rz diag(sa^2, sb^2) Rz^T + eps I.  Its profile, with the inverse taken by
    numpy.linalg.inv, must match the render (pins the conic and the quadratic form's cross term)."""
    f, z, o = 90.0, 3.0, 0.7
    ls = [-2.2, -3.0, -2.6]
    cam = pinhole(64, 64, f=f, cx=32.5, cy=32.5)
    c, s = np.cos(np.pi / 8), np.sin(np.pi / 8)  # quaternion of a 45 degree turn about z
    sc = scene_from([[0, 0, z]], [ls], [[c, 0, 0, s]], [logit(o)], [[1, 1, 1]], [cam])
    r = render(oracle_mod, sc, sc.settings())
    sa, sb = np.exp(widen(ls[0])), np.exp(widen(ls[1]))
    q32 = np.float32([c, 0, 0, s]).astype(float)
    th = 2 * np.arctan2(q32[3], q32[0])
    Rz = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]])
    cov = (f / z) ** 2 * Rz @ np.diag([sa ** 2, sb ** 2]) @ Rz.T + widen(0.3) * np.eye(2)
    assert abs(cov[0, 1]) > 1.0
    inv = np.linalg.inv(cov)
    ys, xs = np.mgrid[0:64, 0:64]
    d = np.stack([xs + 0.5 - 32.5, ys + 0.5 - 32.5], -1)
    qf = np.einsum("...i,ij,...j->...", d, inv, d)
    o32 = 1 / (1 + np.exp(-widen(logit(o))))
    alpha = np.minimum(widen(0.99), o32 * np.exp(-0.5 * qf))
    alpha = np.where(alpha >= widen(1 / 255), alpha, 0.0)
    np.testing.assert_allclose(r["fwd"]["T_final"], 1 - alpha, rtol=1e-9, atol=1e-11)


def test_evaluation_counts(oracle_mod):
    """E_tile (every list entry a pixel walks up to its stop) and E_box (those whose exact
    alpha_min box holds the pixel): for one Gaussian, E_tile = the pixels of its tiles and
    E_box = the pixel centres inside the box sqrt(2 ln(o / alpha_min) Sigma'_xx) x (..yy) around
    its centre; on a scene, blends <= E_box <= E_tile."""
    cam = pinhole(64, 64, f=80.0, cx=29.3, cy=35.1)
    sc = scene_from([[0.1, -0.05, 3.0]], [[-2.3, -2.8, -2.5]], [[0.9, 0.2, -0.3, 0.1]], [logit(0.7)], [[1, 1, 1]],
                    [cam])
    st = sc.settings()
    r = render(oracle_mod, sc, st)
    rec = r["rec"]
    (tx0, ty0, tx1, ty1) = rec["rect"][0]
    assert r["fwd"]["n_evaluated"] == (tx1 - tx0 + 1) * (ty1 - ty0 + 1) * 256
    A, B, C = rec["conic"][0]
    det = A * C - B * B
    Q = 2 * math.log(rec["opacity"][0] / widen(1 / 255))
    ys, xs = np.mgrid[0:64, 0:64]
    dx, dy = xs + 0.5 - rec["mean2d"][0, 0], ys + 0.5 - rec["mean2d"][0, 1]
    in_tiles = (xs // 16 >= tx0) & (xs // 16 <= tx1) & (ys // 16 >= ty0) & (ys // 16 <= ty1)
    box = (dx * dx <= Q * C / det) & (dy * dy <= Q * A / det) & in_tiles
    assert r["fwd"]["n_box"] == int(box.sum()) > 0
    sc2 = scenes.random_scene(2000, 96, 80, seed=4, log_scale_mean=-2.6, opacity_std=1.5)
    f = render(oracle_mod, sc2, sc2.settings())["fwd"]
    assert 0 < f["n_blended"] <= f["n_box"] <= f["n_evaluated"]
