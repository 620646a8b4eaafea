"""Pins of the oracle's composition of partial renders (CPU)."""
import numpy as np

import oracle
from helpers import depth_layered_scene, subset


def _forward(scene, settings):
    out = oracle.iteration(scene, settings, backward=False)
    return (np.stack([o["fwd"]["image"] for o in out]), np.stack([o["fwd"]["T_final"] for o in out]))


def test_depth_separated_subsets_compose_to_the_union():
    sc, layers = depth_layered_scene(60, 48, 40, seed=3, layers=((2.0, 3.0), (4.0, 5.0), (6.5, 8.0)))
    bg = (0.2, 0.5, 0.9)
    full_img, full_T = _forward(sc, sc.settings(t_min=0.0, bg=bg))
    parts = [_forward(subset(sc, idx), sc.settings(t_min=0.0)) for idx in layers]
    # the renderer's constants are float32 values
    img, T = oracle.compose([p[0] for p in parts], [p[1] for p in parts], [float(np.float32(x)) for x in bg])
    assert full_T.min() < 0.9  # the layers overlap on screen
    assert np.allclose(img, full_img, rtol=0, atol=1e-12)
    assert np.allclose(T, full_T, rtol=0, atol=1e-12)


def test_overlapping_depths_do_not_compose_exactly():
    # the same subsets interleaved in depth: composition is not the union's compositing
    sc, layers = depth_layered_scene(60, 48, 40, seed=4, layers=((2.0, 6.0), (2.0, 6.0)))
    full_img, _ = _forward(sc, sc.settings(t_min=0.0))
    parts = [_forward(subset(sc, idx), sc.settings(t_min=0.0)) for idx in layers]
    img, _ = oracle.compose([p[0] for p in parts], [p[1] for p in parts], (0, 0, 0))
    assert np.abs(img - full_img).max() > 1e-3


def test_transparent_partial_is_an_identity_and_composition_is_associative():
    rng = np.random.default_rng(0)
    V, H, W = 2, 5, 7
    mk = lambda: (rng.random((V, 3, H, W)) * 0.5, rng.random((V, H, W)))
    a, b, c = mk(), mk(), mk()
    clear = (np.zeros((V, 3, H, W)), np.ones((V, H, W)))
    bg = (0.3, 0.1, 0.7)
    ref = oracle.compose([a[0], b[0], c[0]], [a[1], b[1], c[1]], bg)
    with_clear = oracle.compose([a[0], clear[0], b[0], c[0], clear[0]], [a[1], clear[1], b[1], c[1], clear[1]], bg)
    assert np.array_equal(ref[0], with_clear[0]) and np.array_equal(ref[1], with_clear[1])
    ab = oracle.compose([a[0], b[0]], [a[1], b[1]], (0, 0, 0))
    nested = oracle.compose([ab[0], c[0]], [ab[1], c[1]], bg)
    assert np.allclose(nested[0], ref[0], rtol=0, atol=1e-14) and np.allclose(nested[1], ref[1], rtol=0, atol=1e-15)
    one = oracle.compose([a[0]], [a[1]], bg)
    assert np.allclose(one[0], a[0] + a[1][:, None] * np.asarray(bg).reshape(1, 3, 1, 1), rtol=0, atol=1e-15)
