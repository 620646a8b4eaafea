"""Small builders shared by the tests (inputs only; no rendering arithmetic)."""
import numpy as np

from differentiable_raster_amd import scenes


def scene_from(means, log_scales, quats, logits, dc, cams, sh_rest=None, sh_degree=0, target=None, dldc=None):
    """A Scene from per-Gaussian rows: means (n,3), log_scales (n,3), quats (n,4) wxyz,
    logits (n,), dc (n,3); sh_rest (n, 3*((d+1)^2-1)) in (k*3+ch) order without the DC."""
    means = np.asarray(means, np.float32).reshape(-1, 3)
    n = means.shape[0]
    k = (sh_degree + 1) ** 2
    sh = np.zeros((3 * k, n), np.float32)
    sh[0:3] = np.asarray(dc, np.float32).reshape(n, 3).T
    if sh_rest is not None:
        sh[3:] = np.asarray(sh_rest, np.float32).reshape(n, 3 * (k - 1)).T
    V = len(cams)
    H, W = cams[0].height, cams[0].width
    loss = "l1" if dldc is None else "external"
    if target is None and dldc is None:
        target = np.zeros((V, 3, H, W), np.float32)
    return scenes.Scene(
        name="handmade",
        means=np.ascontiguousarray(means.T),
        log_scales=np.ascontiguousarray(np.asarray(log_scales, np.float32).reshape(n, 3).T),
        quats=np.ascontiguousarray(np.asarray(quats, np.float32).reshape(n, 4).T),
        opacity_logits=np.asarray(logits, np.float32).reshape(n),
        sh=sh, sh_degree=sh_degree, cameras=list(cams), loss=loss,
        target=None if target is None else np.asarray(target, np.float32),
        dldc=None if dldc is None else np.asarray(dldc, np.float32))


def pinhole(width, height, f=None, cx=None, cy=None, R=None, t=None, fy=None):
    """A camera with explicit intrinsics (float32 values) and optional pose."""
    cam = scenes.identity_camera(width, height)
    if f is not None:
        cam.fx = cam.fy = float(np.float32(f))
    if fy is not None:
        cam.fy = float(np.float32(fy))
    if cx is not None:
        cam.cx = float(np.float32(cx))
    if cy is not None:
        cam.cy = float(np.float32(cy))
    if R is not None:
        cam.R = np.asarray(R, np.float32)
        cam.t = np.asarray(t, np.float32)
        Rd = cam.R.astype(np.float64)
        cam.campos = (-Rd.T @ cam.t.astype(np.float64)).astype(np.float32)
    return cam


def logit(o):
    return float(np.log(o / (1.0 - o)))


def subset(scene, idx, name=None):
    """The scene restricted to the Gaussians idx (same cameras, target and dL/dpixel)."""
    idx = np.asarray(idx)
    return scenes.Scene(
        name=name or f"{scene.name}-subset", means=np.ascontiguousarray(scene.means[:, idx]),
        log_scales=np.ascontiguousarray(scene.log_scales[:, idx]), quats=np.ascontiguousarray(scene.quats[:, idx]),
        opacity_logits=np.ascontiguousarray(scene.opacity_logits[idx]), sh=np.ascontiguousarray(scene.sh[:, idx]),
        sh_degree=scene.sh_degree, cameras=scene.cameras, loss=scene.loss, target=scene.target, dldc=scene.dldc)


def depth_layered_scene(n_per_layer, width, height, seed, layers=((2.0, 3.0), (5.0, 7.0)), views=1):
    """A scene whose Gaussians come in depth layers (layer i entirely in front of layer i + 1 for
    the identity-posed and slightly moved test cameras); returns (scene, index arrays per layer)."""
    parts = [scenes.random_scene(n_per_layer, width, height, seed + 17 * i, views=views, z_range=z,
                                 log_scale_mean=-3.0) for i, z in enumerate(layers)]
    first = parts[0]
    cat = lambda f: np.ascontiguousarray(np.concatenate([getattr(p, f) for p in parts], axis=-1))
    sc = scenes.Scene(name=f"layers-{len(layers)}x{n_per_layer}-{width}x{height}-s{seed}", means=cat("means"),
                      log_scales=cat("log_scales"), quats=cat("quats"), opacity_logits=cat("opacity_logits"),
                      sh=cat("sh"), sh_degree=first.sh_degree, cameras=first.cameras, loss=first.loss,
                      target=first.target, dldc=first.dldc)
    idx = [np.arange(i * n_per_layer, (i + 1) * n_per_layer) for i in range(len(layers))]
    return sc, idx
