"""Seeded synthetic workloads for tile-based differentiable 3D Gaussian splatting.

This module only draws inputs: Gaussian parameters, pinhole cameras, loss targets and the
render settings a workload runs with.  It holds none of the rendering arithmetic, so both the
HIP path and the CPU oracle can take their inputs from it without sharing any of the method.

The pages evaluate on real captures (six unnamed datasets in ByteSplat, arXiv 2610.02851,
English abstract; Rubble in Grendel, arXiv 2406.18533, experiments; "large-scale datasets" in
GS-Scale, arXiv 2509.15645, and Splaxel, arXiv 2606.18588, English abstracts).  None is
available, so five seeded synthetic scenes stand in for them, with the sizes, distributions
and camera layouts listed in ``CONFIGS``.  Every draw uses ``numpy.random.Generator(PCG64(seed))``
with seed ``1000 + config`` in a fixed order: means, log-scales, quaternions, opacity logits,
SH coefficients, cameras, then the target image or the supplied per-pixel loss gradient.

Layouts (structure of arrays, float32):
  means[3][N], log_scales[3][N], quats[4][N] (w, x, y, z), opacity_logits[N],
  sh[3*(d+1)^2][N] with row index k*3 + channel for SH coefficient k.
Cameras: world-to-camera rotation R (row-major 3x3) and translation t, OpenCV axes
(x right, y down, z forward), focal lengths in pixels, principal point in pixels, and the
camera centre in world coordinates.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

TILE = 16


@dataclasses.dataclass
class Camera:
    width: int
    height: int
    fx: float
    fy: float
    cx: float
    cy: float
    R: np.ndarray       # (3, 3) float32, world -> camera rotation, row-major
    t: np.ndarray       # (3,) float32, world -> camera translation
    campos: np.ndarray  # (3,) float32, camera centre in world coordinates

    @property
    def tiles_x(self) -> int:
        return (self.width + TILE - 1) // TILE

    @property
    def tiles_y(self) -> int:
        return (self.height + TILE - 1) // TILE

    @property
    def n_tiles(self) -> int:
        return self.tiles_x * self.tiles_y


@dataclasses.dataclass
class RenderSettings:
    """Constants of the method that the pages leave open (readings, not page values)."""
    znear: float = 0.2
    eps2d: float = 0.3
    alpha_min: float = 1.0 / 255.0
    alpha_max: float = 0.99
    t_min: float = 1e-4
    bg: tuple = (0.0, 0.0, 0.0)
    sh_degree: int = 3
    tile_cap: int = 0


@dataclasses.dataclass
class Scene:
    name: str
    means: np.ndarray
    log_scales: np.ndarray
    quats: np.ndarray
    opacity_logits: np.ndarray
    sh: np.ndarray
    sh_degree: int
    cameras: list
    loss: str                       # "l1" (target given) or "external" (dL/dpixel given)
    target: Optional[np.ndarray]    # (V, 3, H, W) float32 or None
    dldc: Optional[np.ndarray]      # (V, 3, H, W) float32 or None

    @property
    def n(self) -> int:
        return int(self.means.shape[1])

    def settings(self, **kw) -> RenderSettings:
        s = RenderSettings(sh_degree=self.sh_degree)
        for k, v in kw.items():
            setattr(s, k, v)
        return s


CONFIGS = {
    1: "tiny: 4096 Gaussians, 128x128, 1 view, SH degree 0, L1 vs U(0,1) target",
    2: "100K Gaussians, 1280x720, 1 view, SH degree 3, supplied dL/dpixel",
    3: "1M Gaussians in 64 blobs, 1920x1080, 4 ring views, SH degree 3, L1",
    4: "the 1M-Gaussian scene with a per-tile cap K in {256, 512, 1024}",
    5: "40M Gaussians on a city-like ground grid, 3840x2160, 4 views, SH degree 3, L1",
}


def focal_for_fov_x(width: int, fov_x_deg: float = 60.0) -> float:
    return (width / 2.0) / math.tan(math.radians(fov_x_deg) / 2.0)


def camera_from_rows(width, height, x_axis, y_axis, z_axis, position, fov_x_deg=60.0) -> Camera:
    """Pinhole camera whose camera-frame axes are the given world directions (float64 in)."""
    R = np.stack([x_axis, y_axis, z_axis]).astype(np.float64)
    p = np.asarray(position, dtype=np.float64)
    t = -R @ p
    f = focal_for_fov_x(width, fov_x_deg)
    return Camera(width=width, height=height, fx=float(np.float32(f)), fy=float(np.float32(f)),
                  cx=float(np.float32(width / 2.0)), cy=float(np.float32(height / 2.0)),
                  R=R.astype(np.float32), t=t.astype(np.float32), campos=p.astype(np.float32))


def identity_camera(width: int, height: int, fov_x_deg: float = 60.0) -> Camera:
    e = np.eye(3)
    return camera_from_rows(width, height, e[0], e[1], e[2], np.zeros(3), fov_x_deg)


def look_at_camera(width, height, position, target, down_hint, fov_x_deg=60.0) -> Camera:
    p = np.asarray(position, np.float64)
    z = np.asarray(target, np.float64) - p
    z /= np.linalg.norm(z)
    d = np.asarray(down_hint, np.float64)
    y = d - np.dot(d, z) * z
    y /= np.linalg.norm(y)
    x = np.cross(y, z)
    return camera_from_rows(width, height, x, y, z, p, fov_x_deg)


def _unit_quats(rng, n):
    q = rng.standard_normal((4, n), dtype=np.float32)
    norm = np.sqrt((q.astype(np.float64) ** 2).sum(0))
    norm[norm == 0] = 1.0
    return (q / norm).astype(np.float32)


def _sh(rng, n, degree, rest_sigma=0.2):
    k = (degree + 1) ** 2
    sh = np.empty((3 * k, n), np.float32)
    sh[0:3] = rng.random((3, n), dtype=np.float32)
    if k > 1:
        sh[3:] = rng.standard_normal((3 * (k - 1), n), dtype=np.float32) * np.float32(rest_sigma)
    return sh


def make_scene(cfg: int, seed: Optional[int] = None) -> Scene:
    """The synthetic stand-in for workload ``cfg`` (1..5; 4 is scene 3, the cap is a setting)."""
    if cfg == 4:
        cfg_draw = 3
    else:
        cfg_draw = cfg
    rng = np.random.Generator(np.random.PCG64(1000 + cfg if seed is None else seed))
    f32 = np.float32
    if cfg_draw == 1:
        n, W, H, V, deg = 4096, 128, 128, 1, 0
        means = np.empty((3, n), f32)
        means[0:2] = rng.uniform(-1, 1, (2, n)).astype(f32)
        means[2] = rng.uniform(2, 6, n).astype(f32)
        log_scales = (rng.standard_normal((3, n), dtype=f32) * f32(0.5) - f32(3.0)).astype(f32)
        quats = _unit_quats(rng, n)
        opac = rng.standard_normal(n, dtype=f32)
        sh = _sh(rng, n, deg)
        cams = [identity_camera(W, H)]
        target = rng.random((V, 3, H, W), dtype=f32)
        return Scene("tiny-4k-128", means, log_scales, quats, opac, sh, deg, cams, "l1", target, None)
    if cfg_draw == 2:
        n, W, H, V, deg = 100_000, 1280, 720, 1, 3
        means = np.empty((3, n), f32)
        means[0:2] = rng.uniform(-10, 10, (2, n)).astype(f32)
        means[2] = rng.uniform(1, 30, n).astype(f32)
        log_scales = (rng.standard_normal((3, n), dtype=f32) * f32(0.7) - f32(4.0)).astype(f32)
        quats = _unit_quats(rng, n)
        opac = rng.standard_normal(n, dtype=f32)
        sh = _sh(rng, n, deg)
        cams = [identity_camera(W, H)]
        s = (rng.integers(0, 2, (V, 3, H, W)) * 2 - 1).astype(f32)
        g = rng.standard_normal((V, 3, H, W), dtype=f32)
        dldc = (f32(0.8) * s + f32(0.2) * g).astype(f32)
        return Scene("100k-720p", means, log_scales, quats, opac, sh, deg, cams, "external", None, dldc)
    if cfg_draw == 3:
        n, W, H, V, deg = 1_000_000, 1920, 1080, 4, 3
        n_blobs = 64
        centres = np.empty((3, n_blobs), f32)
        centres[0:2] = rng.uniform(-20, 20, (2, n_blobs)).astype(f32)
        centres[2] = rng.uniform(1, 50, n_blobs).astype(f32)
        blob = np.arange(n) // (n // n_blobs)
        means = (centres[:, blob] + rng.standard_normal((3, n), dtype=f32) * f32(0.5)).astype(f32)
        log_scales = (rng.standard_normal((3, n), dtype=f32) * f32(0.8) - f32(4.5)).astype(f32)
        quats = _unit_quats(rng, n)
        opac = (rng.standard_normal(n, dtype=f32) * f32(1.5)).astype(f32)
        sh = _sh(rng, n, deg)
        centre = np.array([0.0, 0.0, 25.5])
        cams = []
        for _ in range(V):
            a = rng.uniform(0.0, 2.0 * math.pi)
            pos = centre + 45.0 * np.array([math.sin(a), 0.0, -math.cos(a)])
            cams.append(look_at_camera(W, H, pos, centre, (0.0, 1.0, 0.0)))
        target = rng.random((V, 3, H, W), dtype=f32)
        return Scene("1m-blobs-1080p-4v", means, log_scales, quats, opac, sh, deg, cams, "l1", target, None)
    if cfg_draw == 5:
        n, W, H, V, deg = 40_000_000, 3840, 2160, 4, 3
        width = 6325
        cell = np.arange(n, dtype=np.int64)
        means = np.empty((3, n), f32)
        means[0] = ((cell % width).astype(np.float64) * 0.1 - 316.25).astype(f32)
        means[1] = ((cell // width).astype(np.float64) * 0.1 - 316.25).astype(f32)
        del cell
        means[0:2] += rng.random((2, n), dtype=f32) * f32(0.1)
        means[2] = rng.exponential(10.0, n).astype(f32)
        log_scales = (rng.standard_normal((3, n), dtype=f32) - f32(5.0)).astype(f32)
        quats = _unit_quats(rng, n)
        opac = rng.standard_normal(n, dtype=f32)
        sh = _sh(rng, n, deg)
        cams = []
        pitch = math.radians(45.0)
        for _ in range(V):
            x0, y0 = rng.uniform(-158.0, 158.0, 2)
            yaw = rng.uniform(0.0, 2.0 * math.pi)
            fwd = np.array([math.cos(pitch) * math.cos(yaw), math.cos(pitch) * math.sin(yaw), -math.sin(pitch)])
            pos = np.array([x0, y0, 100.0])
            cams.append(look_at_camera(W, H, pos, pos + fwd, (0.0, 0.0, -1.0)))
        target = rng.random((V, 3, H, W), dtype=f32)
        return Scene("40m-city-4k-4v", means, log_scales, quats, opac, sh, deg, cams, "l1", target, None)
    raise ValueError(f"unknown workload {cfg}")


def random_scene(n: int, width: int, height: int, seed: int, *, views: int = 1, sh_degree: int = 0,
                 z_range=(2.0, 6.0), xy_extent=1.0, log_scale_mean=-3.0, log_scale_std=0.5,
                 opacity_std=1.0, loss: str = "l1") -> Scene:
    """A small seeded scene in front of identity-posed cameras (for tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f32 = np.float32
    means = np.empty((3, n), f32)
    means[0:2] = rng.uniform(-xy_extent, xy_extent, (2, n)).astype(f32)
    means[2] = rng.uniform(z_range[0], z_range[1], n).astype(f32)
    log_scales = (rng.standard_normal((3, n), dtype=f32) * f32(log_scale_std) + f32(log_scale_mean)).astype(f32)
    quats = _unit_quats(rng, n)
    opac = (rng.standard_normal(n, dtype=f32) * f32(opacity_std)).astype(f32)
    sh = _sh(rng, n, sh_degree)
    cams = []
    for v in range(views):
        if v == 0:
            cams.append(identity_camera(width, height))
        else:
            a = rng.uniform(-0.3, 0.3)
            pos = np.array([rng.uniform(-0.5, 0.5), rng.uniform(-0.5, 0.5), rng.uniform(-0.5, 0.0)])
            tgt = np.array([math.sin(a) * 4.0, 0.0, 4.0])
            cams.append(look_at_camera(width, height, pos, tgt, (0.0, 1.0, 0.0)))
    target = dldc = None
    if loss == "l1":
        target = rng.random((views, 3, height, width), dtype=f32)
    else:
        s = (rng.integers(0, 2, (views, 3, height, width)) * 2 - 1).astype(f32)
        dldc = (f32(0.8) * s + f32(0.2) * rng.standard_normal((views, 3, height, width), dtype=f32)).astype(f32)
    return Scene(f"random-{n}-{width}x{height}-s{seed}", means, log_scales, quats, opac, sh, sh_degree,
                 cams, loss, target, dldc)
