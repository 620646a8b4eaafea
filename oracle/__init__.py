"""CPU oracle for tile-based differentiable 3D Gaussian splatting (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  It never imports the HIP library or its binding, and the HIP library never
imports it.  The per-Gaussian projection and the per-pixel compositing and backward are
plain double-precision C (``gs_oracle.c``); binning is plain NumPy (a cumulative sum, an
enumeration and a stable sort).

What the method computes is never written out on the pages: ByteSplat (arXiv 2610.02851,
English abstract) names forward and backward rasterization, their fusion and a per-tile
pruning; Grendel (arXiv 2406.18533, English abstract) notes that each Gaussian touches a small
subset of pixels and trains on batches of views; GS-Scale (arXiv 2509.15645, English abstract)
adds per-view frustum culling.  The formulas are the plainest reading of EWA splatting with
front-to-back alpha compositing; the constants are readings and arrive as parameters.
Parity status per function is stated in each docstring.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gs_oracle.c")
# GS_ORACLE_LIB names another build of gs_oracle.c to load (the sanitizer test's).
_LIB = os.environ.get("GS_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the C part of the oracle (gcc, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-std=c11", "-Wall",
                               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out_dir: str) -> str:
    """out_dir/liboracle_san.so: the oracle under gcc's AddressSanitizer and
    UndefinedBehaviorSanitizer (load it with gcc's libasan preloaded and GS_ORACLE_LIB set)."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fopenmp", "-ffp-contract=off", "-std=c11", "-Wall",
                           "-shared", "-fPIC", _SRC, "-o", lib, "-lm"])
    return lib


class _Camera(ctypes.Structure):
    _fields_ = [("width", ctypes.c_int32), ("height", ctypes.c_int32),
                ("fx", ctypes.c_double), ("fy", ctypes.c_double),
                ("cx", ctypes.c_double), ("cy", ctypes.c_double),
                ("R", ctypes.c_double * 9), ("t", ctypes.c_double * 3),
                ("campos", ctypes.c_double * 3)]


class _Params(ctypes.Structure):
    _fields_ = [("znear", ctypes.c_double), ("eps2d", ctypes.c_double),
                ("alpha_min", ctypes.c_double), ("alpha_max", ctypes.c_double),
                ("t_min", ctypes.c_double), ("bg", ctypes.c_double * 3),
                ("sh_degree", ctypes.c_int32), ("tile", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=False)
        _lib = ctypes.CDLL(_LIB)
        _lib.orc_sh_basis.restype = None
        _lib.orc_project.restype = None
        _lib.orc_project_f64.restype = None
        _lib.orc_project_backward.restype = None
        _lib.orc_project_backward_errbound.restype = None
        _lib.orc_sh_basis_grad.restype = None
        _lib.orc_raster_forward.restype = None
        _lib.orc_raster_backward.restype = None
        _lib.orc_raster_bruteforce.restype = None
        _lib.orc_pair_alpha.restype = None
        _lib.orc_num_threads.restype = ctypes.c_int
        _lib.orc_set_num_threads.restype = None
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Set the OpenMP threads of the oracle's parallel loops."""
    _load().orc_set_num_threads(ctypes.c_int(int(n)))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x) -> float:
    """Constants reach both implementations as float32 values; the oracle widens them."""
    return float(np.float32(x))


def _cam(c) -> _Camera:
    cam = _Camera()
    cam.width, cam.height = int(c.width), int(c.height)
    cam.fx, cam.fy, cam.cx, cam.cy = _f32(c.fx), _f32(c.fy), _f32(c.cx), _f32(c.cy)
    R = np.asarray(c.R, np.float32).astype(np.float64).reshape(9)
    t = np.asarray(c.t, np.float32).astype(np.float64).reshape(3)
    cp = np.asarray(c.campos, np.float32).astype(np.float64).reshape(3)
    for k in range(9):
        cam.R[k] = R[k]
    for k in range(3):
        cam.t[k] = t[k]
        cam.campos[k] = cp[k]
    return cam


def _params(s, tile: int = 16) -> _Params:
    p = _Params()
    p.znear, p.eps2d = _f32(s.znear), _f32(s.eps2d)
    p.alpha_min, p.alpha_max, p.t_min = _f32(s.alpha_min), _f32(s.alpha_max), _f32(s.t_min)
    for k in range(3):
        p.bg[k] = _f32(s.bg[k])
    p.sh_degree = int(s.sh_degree)
    p.tile = tile
    return p


# ---------------------------------------------------------------------------------------
# Spherical harmonics
# ---------------------------------------------------------------------------------------
def sh_basis(degree: int, dirs: np.ndarray) -> np.ndarray:
    """Real orthonormal SH basis values Y[l*l+l+m] at unit directions dirs (n, 3).

    Parity: pinned against scipy's complex spherical harmonics (converted to real form) and
    by quadrature orthonormality."""
    lib = _load()
    dirs = np.ascontiguousarray(dirs, np.float64)
    out = np.zeros((dirs.shape[0], 16), np.float64)
    for i in range(dirs.shape[0]):
        lib.orc_sh_basis(ctypes.c_int(degree), _p(dirs[i]), _p(out[i]))
    return out[:, : (degree + 1) ** 2]


# ---------------------------------------------------------------------------------------
# Projection (per view)
# ---------------------------------------------------------------------------------------
def project(scene, cam, settings) -> dict:
    """Project every Gaussian of ``scene`` into camera ``cam`` (no compaction).

    Returns per-Gaussian arrays: visible, mean2d (n,2), cov2d (n,3), conic (n,3), opacity,
    color (n,3), depth, rect (n,4) int32 (tx0, ty0, tx1, ty1), n_tiles, flag.
    Parity: pinned by closed forms (on/off-axis isotropic Gaussians, quaternion axes,
    camera-frame equivalence) and by a brute-force check of the opacity-aware box."""
    lib = _load()
    n = scene.means.shape[1]
    out = dict(visible=np.zeros(n, np.int8), mean2d=np.zeros((n, 2)), cov2d=np.zeros((n, 3)),
               conic=np.zeros((n, 3)), opacity=np.zeros(n), color=np.zeros((n, 3)), depth=np.zeros(n),
               rect=np.zeros((n, 4), np.int32), n_tiles=np.zeros(n, np.int32), flag=np.zeros(n, np.int8))
    arrs = [np.ascontiguousarray(a, np.float32) for a in
            (scene.means, scene.log_scales, scene.quats, scene.opacity_logits, scene.sh)]
    c, pp = _cam(cam), _params(settings)
    lib.orc_project(ctypes.c_int64(n), *[_p(a) for a in arrs], ctypes.byref(c), ctypes.byref(pp),
                    _p(out["visible"]), _p(out["mean2d"]), _p(out["cov2d"]), _p(out["conic"]),
                    _p(out["opacity"]), _p(out["color"]), _p(out["depth"]), _p(out["rect"]),
                    _p(out["n_tiles"]), _p(out["flag"]))
    return out


def sh_basis_grad(degree: int, dirs: np.ndarray) -> np.ndarray:
    """Cartesian gradients (n, 16, 3) of the basis polynomials of ``sh_basis`` at dirs (n, 3).

    Parity: pinned by central finite differences of ``sh_basis`` (itself pinned against scipy)."""
    lib = _load()
    dirs = np.ascontiguousarray(dirs, np.float64)
    out = np.zeros((dirs.shape[0], 16, 3), np.float64)
    for i in range(dirs.shape[0]):
        lib.orc_sh_basis_grad(ctypes.c_int(degree), _p(dirs[i]), _p(out[i]))
    return out[:, : (degree + 1) ** 2]


def scene_params_f64(scene) -> dict:
    """The scene's float32 parameters, widened exactly to float64 (SoA, as the scene holds them)."""
    return dict(means=np.ascontiguousarray(scene.means, np.float64),
                log_scales=np.ascontiguousarray(scene.log_scales, np.float64),
                quats=np.ascontiguousarray(scene.quats, np.float64),
                opacity_logits=np.ascontiguousarray(scene.opacity_logits, np.float64),
                sh=np.ascontiguousarray(scene.sh, np.float64))


_PARAM_KEYS = ("means", "log_scales", "quats", "opacity_logits", "sh")


def project_f64(params: dict, cam, settings) -> dict:
    """``project`` on double-precision parameters (``scene_params_f64`` layout), so that the
    projection can be differentiated numerically.  Same outputs as ``project``."""
    lib = _load()
    n = params["means"].shape[1]
    out = dict(visible=np.zeros(n, np.int8), mean2d=np.zeros((n, 2)), cov2d=np.zeros((n, 3)),
               conic=np.zeros((n, 3)), opacity=np.zeros(n), color=np.zeros((n, 3)), depth=np.zeros(n),
               rect=np.zeros((n, 4), np.int32), n_tiles=np.zeros(n, np.int32), flag=np.zeros(n, np.int8))
    arrs = [np.ascontiguousarray(params[k], np.float64) for k in _PARAM_KEYS]
    c, pp = _cam(cam), _params(settings)
    lib.orc_project_f64(ctypes.c_int64(n), *[_p(a) for a in arrs], ctypes.byref(c), ctypes.byref(pp),
                        _p(out["visible"]), _p(out["mean2d"]), _p(out["cov2d"]), _p(out["conic"]),
                        _p(out["opacity"]), _p(out["color"]), _p(out["depth"]), _p(out["rect"]),
                        _p(out["n_tiles"]), _p(out["flag"]))
    return out


def project_backward(params: dict, cam, settings, visible: np.ndarray, g_mean2d, g_conic, g_opacity, g_color,
                     acc: Optional[dict] = None, error_bound: bool = False) -> dict:
    """Chain rule of the projection for one view (test infrastructure).

    ``params``: ``scene_params_f64`` layout.  ``visible`` (n,) selects the Gaussians; the
    gradients with respect to the 2D outputs are indexed by Gaussian: g_mean2d (n,2),
    g_conic (n,3) for (A, B, C), g_opacity (n,), g_color (n,3).  Adds this view's share to
    ``acc`` (created zeroed when None) and returns it: d_means (3,n), d_log_scales (3,n),
    d_quats (4,n) with respect to the raw quaternion, d_opacity_logits (n,), d_sh (3(d+1)^2, n)
    and flag (n,) = a colour channel's pre-clamp value lies within float32 reach of zero.

    Parity: pinned by central finite differences of ``project_f64`` for every parameter, by
    invariances (an isotropic Gaussian has no quaternion gradient; the quaternion gradient is
    orthogonal to the quaternion) and by closed forms for the colour and opacity terms.

    error_bound: also add e_means, e_log_scales, e_quats, e_opacity_logits, e_sh: a first-order
    running bound on the error of evaluating the same chain in float32 (a tolerance model for
    comparisons, from the rounding of every operation; pinned against float32 evaluations of the
    chain in the tests)."""
    lib = _load()
    n = params["means"].shape[1]
    nk = params["sh"].shape[0]
    if acc is None:
        acc = dict(d_means=np.zeros((3, n)), d_log_scales=np.zeros((3, n)), d_quats=np.zeros((4, n)),
                   d_opacity_logits=np.zeros(n), d_sh=np.zeros((nk, n)), flag=np.zeros(n, np.int8))
    arrs = [np.ascontiguousarray(params[k], np.float64) for k in _PARAM_KEYS]
    vis = np.ascontiguousarray(visible, np.int8)
    g = [np.ascontiguousarray(x, np.float64) for x in (g_mean2d, g_conic, g_opacity, g_color)]
    assert g[0].shape == (n, 2) and g[1].shape == (n, 3) and g[2].shape == (n,) and g[3].shape == (n, 3)
    c, pp = _cam(cam), _params(settings)
    lib.orc_project_backward(ctypes.c_int64(n), *[_p(a) for a in arrs], ctypes.byref(c), ctypes.byref(pp),
                             _p(vis), *[_p(x) for x in g], _p(acc["d_means"]), _p(acc["d_log_scales"]),
                             _p(acc["d_quats"]), _p(acc["d_opacity_logits"]), _p(acc["d_sh"]), _p(acc["flag"]))
    if error_bound:
        for k in ("d_means", "d_log_scales", "d_quats", "d_opacity_logits", "d_sh"):
            acc.setdefault("e" + k[1:], np.zeros_like(acc[k]))
        lib.orc_project_backward_errbound(ctypes.c_int64(n), *[_p(a) for a in arrs], ctypes.byref(c),
                                          ctypes.byref(pp), _p(vis), *[_p(x) for x in g], _p(acc["e_means"]),
                                          _p(acc["e_log_scales"]), _p(acc["e_quats"]), _p(acc["e_opacity_logits"]),
                                          _p(acc["e_sh"]))
    return acc


def compact(proj: dict) -> dict:
    """Visible Gaussians in ascending original index become slots 0..n_vis-1."""
    ids = np.nonzero(proj["visible"])[0].astype(np.int32)
    rec = {k: v[ids] for k, v in proj.items() if k != "visible"}
    rec["vis_ids"] = ids
    rec["vis_count"] = int(ids.size)
    return rec


# ---------------------------------------------------------------------------------------
# Binning (NumPy): scan, emission, stable sort by (tile, depth), ranges, cap
# ---------------------------------------------------------------------------------------
def depth_bits(depth) -> np.ndarray:
    """The depth key is the raw float32 bit pattern of camera-space z (positive, monotone)."""
    return np.asarray(depth, np.float32).view(np.uint32)


def bin_tiles(rect: np.ndarray, n_tiles: np.ndarray, dbits: np.ndarray, tiles_x: int, tiles_y: int) -> dict:
    """Instances of (tile, slot) for each slot's tile rectangle, sorted by (tile, depth, slot).

    offsets = exclusive cumulative sum of n_tiles; slot s emits its tiles row-major at
    offsets[s] + k with key (tile << 32) | depth_bits and value s; a stable sort by key keeps
    equal keys in slot order; ranges[t] = [first, last + 1) of tile t, (0, 0) when empty.
    Parity: pinned by brute-force enumeration and Python's sorted() on tuples."""
    n = int(n_tiles.shape[0])
    n_tiles = n_tiles.astype(np.int64)
    offsets = np.zeros(n, np.int64)
    if n:
        offsets[1:] = np.cumsum(n_tiles)[:-1]
    M = int(n_tiles.sum()) if n else 0
    slot = np.repeat(np.arange(n, dtype=np.int64), n_tiles)
    k = np.arange(M, dtype=np.int64) - np.repeat(offsets, n_tiles)
    tx0, ty0, tx1, ty1 = (rect[:, i].astype(np.int64) for i in range(4))
    w = np.repeat(tx1 - tx0 + 1, n_tiles)
    tx = np.repeat(tx0, n_tiles) + k % np.maximum(w, 1)
    ty = np.repeat(ty0, n_tiles) + k // np.maximum(w, 1)
    tile = ty * tiles_x + tx
    keys = (tile.astype(np.uint64) << np.uint64(32)) | dbits.astype(np.uint64)[slot]
    order = np.argsort(keys, kind="stable")
    keys_sorted = keys[order]
    vals_sorted = slot[order].astype(np.int32)
    T = tiles_x * tiles_y
    ranges = np.zeros((T, 2), np.int32)
    tiles_sorted = (keys_sorted >> np.uint64(32)).astype(np.int64)
    if M:
        starts = np.searchsorted(tiles_sorted, np.arange(T), side="left")
        ends = np.searchsorted(tiles_sorted, np.arange(T), side="right")
        nonempty = ends > starts
        ranges[nonempty, 0] = starts[nonempty]
        ranges[nonempty, 1] = ends[nonempty]
    return dict(offsets=offsets, num_instances=M, keys_emitted=keys, keys=keys_sorted, vals=vals_sorted,
                ranges=ranges)


def cap_score(conic_f32: np.ndarray, opacity_f32: np.ndarray) -> np.ndarray:
    """score = o / sqrt(A*C - B*B) = o * sqrt(det of the dilated 2D covariance), in float32
    with one rounding per operation (no contraction), so that it is a decision both
    implementations take identically from the same float32 records."""
    A = conic_f32[:, 0].astype(np.float32)
    B = conic_f32[:, 1].astype(np.float32)
    C = conic_f32[:, 2].astype(np.float32)
    det = np.subtract(np.multiply(A, C, dtype=np.float32), np.multiply(B, B, dtype=np.float32), dtype=np.float32)
    return np.divide(opacity_f32.astype(np.float32), np.sqrt(det, dtype=np.float32), dtype=np.float32)


def cap_tiles(ranges: np.ndarray, vals: np.ndarray, score: np.ndarray, dbits: np.ndarray, K: int) -> dict:
    """Per-tile cap (ByteSplat, arXiv 2610.02851, English abstract: pruning under per-tile
    on-chip memory limits): in a tile with more than K entries keep the K best by
    (score desc, depth asc, slot asc) and leave them in their depth order.
    Parity: pinned by K >= longest list (identity), K = 1 (per-tile argmax) and a Python sort."""
    T = ranges.shape[0]
    out_vals = []
    out_ranges = np.zeros((T, 2), np.int32)
    pos = 0
    for t in range(T):
        s, e = int(ranges[t, 0]), int(ranges[t, 1])
        lst = vals[s:e]
        if e - s > K:
            sc = score[lst]
            d = dbits[lst]
            order = np.lexsort((lst, d, -sc))  # last key is primary
            keep = np.sort(order[:K])
            lst = lst[keep]
        if lst.size:
            out_ranges[t] = (pos, pos + lst.size)
            out_vals.append(lst)
            pos += lst.size
    vals_k = np.concatenate(out_vals).astype(np.int32) if out_vals else np.zeros(0, np.int32)
    return dict(vals=vals_k, ranges=out_ranges, num_instances=int(vals_k.size))


# ---------------------------------------------------------------------------------------
# Rasterization
# ---------------------------------------------------------------------------------------
def _rec(records: dict):
    return [np.ascontiguousarray(records[k], np.float64) for k in ("mean2d", "conic", "opacity", "color")]


def raster_forward(width: int, height: int, ranges: np.ndarray, vals: np.ndarray, records: dict, settings) -> dict:
    """Front-to-back compositing of every pixel over its tile's list.

    Per pixel: alpha = min(alpha_max, o exp(-q/2)); skip alpha < alpha_min; stop before a
    blend that takes T below t_min; C += alpha T c; T *= 1 - alpha; finally C += T bg.
    Returns image (3,H,W), T_final (H,W), n_contrib (H,W), the pair counts n_evaluated (every
    list entry up to the pixel's stop: E_tile), n_blended, n_clamped and n_box (of the evaluated,
    those whose exact alpha_min box holds the pixel: E_box), and the float32 error model used by comparisons: err_C (3,H,W) absolute and
    err_T (H,W) relative bounds; n_dec (H,W) = flagged alpha_min / t_min decisions of the pixel
    (within float32 reach of their threshold), -1 when more than three; flag = n_dec != 0;
    unresolved = n_dec < 0; alt = the pixel under every combination of its flagged decisions
    taken the other way: dict(pix (k,) = y W + x, C (k,3), T (k,), nc (k,)).
    Parity: pinned by the single-Gaussian profile, telescoping identities, a two-Gaussian
    closed form and brute-force all-Gaussians-per-pixel compositing; the error model by
    float32 evaluations of the same compositing."""
    lib = _load()
    image = np.zeros((3, height, width))
    T = np.zeros((height, width))
    nc = np.zeros((height, width), np.int32)
    flag = np.zeros((height, width), np.int8)
    err = np.zeros((3, height, width))
    err_T = np.zeros((height, width))
    counters = np.zeros(4, np.int64)
    ranges = np.ascontiguousarray(ranges, np.int32)
    vals = np.ascontiguousarray(vals, np.int32)
    pp = _params(settings)
    m, c, o, col = _rec(records)
    cap = 4096 + (width * height) // 64
    while True:
        alt_n = np.zeros(1, np.int64)
        alt_pix = np.zeros(cap, np.int64)
        alt_C = np.zeros((cap, 3))
        alt_T = np.zeros(cap)
        alt_nc = np.zeros(cap, np.int32)
        lib.orc_raster_forward(ctypes.c_int32(width), ctypes.c_int32(height), _p(ranges), _p(vals), _p(m), _p(c),
                               _p(o), _p(col), ctypes.byref(pp), _p(image), _p(T), _p(nc), _p(flag), _p(err),
                               _p(err_T), ctypes.c_int64(cap), _p(alt_n), _p(alt_pix), _p(alt_C), _p(alt_T),
                               _p(alt_nc), _p(counters))
        if int(alt_n[0]) <= cap:
            break
        cap = int(alt_n[0])
    k = int(alt_n[0])
    order = np.argsort(alt_pix[:k], kind="stable")
    alt = dict(pix=alt_pix[:k][order], C=alt_C[:k][order], T=alt_T[:k][order], nc=alt_nc[:k][order])
    return dict(image=image, T_final=T, n_contrib=nc, n_dec=flag, flag=flag != 0, unresolved=flag < 0, err_C=err,
                err_T=err_T, alt=alt, n_evaluated=int(counters[0]), n_blended=int(counters[1]),
                n_clamped=int(counters[2]), n_box=int(counters[3]))


def loss_grad_l1(image: np.ndarray, target: np.ndarray, scale: float, err_C: Optional[np.ndarray] = None):
    """dL/dC of L = scale * sum |C - target|: scale * sign(C - target), sign(0) = 0.
    Also returns dg (3,H,W): 2 |scale| for the components whose sign float32 evaluation could
    take differently (|C - target| within the colour's error bound err_C), 0 elsewhere: the
    most that such a component of dL/dC can differ by."""
    diff = image - target.astype(np.float64)
    g = np.sign(diff) * scale
    dg = None
    if err_C is not None:
        dg = np.where(np.abs(diff) <= err_C, 2.0 * abs(scale), 0.0)
    return g, dg


def raster_backward(width: int, height: int, ranges: np.ndarray, vals: np.ndarray, records: dict, settings,
                    dldc: np.ndarray, dg: Optional[np.ndarray] = None) -> dict:
    """Gradients of L with respect to the per-slot 2D records (means2D in pixels, conic
    (A, B, C), activated opacity, post-clamp colour), by reverse traversal of each pixel's
    blended entries.  Returns d_mean2d (S,2), d_conic (S,3), d_opacity (S,), d_color (S,3) and,
    per slot and component (mean x, y, conic A, B, C, opacity, colour r, g, b): mag (S,9) =
    summed magnitudes of the contributions' parts; err (S,9) = summed float32 error bounds of
    the contributions; widen (S,9) = the most that taking flagged decisions the other way (and
    the dL/dC uncertainty dg, optional (3,H,W)) changes the slot's gradient; slot_flag (S,) =
    slots of unresolved pixels; stats = (pixels with flagged decisions, unresolved pixels,
    alternative walks).
    Parity: pinned by central finite differences of the loss and closed-form derivatives; the
    error bounds by float32 evaluations of the same backward."""
    lib = _load()
    S = records["opacity"].shape[0]
    out = dict(d_mean2d=np.zeros((S, 2)), d_conic=np.zeros((S, 3)), d_opacity=np.zeros(S), d_color=np.zeros((S, 3)),
               mag=np.zeros((S, 9)), err=np.zeros((S, 9)), widen=np.zeros((S, 9)), slot_flag=np.zeros(S, np.int8))
    stats = np.zeros(3, np.int64)
    ranges = np.ascontiguousarray(ranges, np.int32)
    vals = np.ascontiguousarray(vals, np.int32)
    dldc = np.ascontiguousarray(dldc, np.float64)
    dgc = None if dg is None else np.ascontiguousarray(dg, np.float64)
    pp = _params(settings)
    m, c, o, col = _rec(records)
    lib.orc_raster_backward(ctypes.c_int32(width), ctypes.c_int32(height), _p(ranges), _p(vals), _p(m), _p(c), _p(o),
                            _p(col), ctypes.byref(pp), _p(dldc), None if dgc is None else _p(dgc),
                            _p(out["d_mean2d"]), _p(out["d_conic"]), _p(out["d_opacity"]), _p(out["d_color"]),
                            _p(out["mag"]), _p(out["err"]), _p(out["widen"]), _p(out["slot_flag"]), _p(stats))
    out["slot_flag"] = out["slot_flag"].astype(bool)
    out["stats"] = dict(flagged_pixels=int(stats[0]), unresolved_pixels=int(stats[1]), alternative_walks=int(stats[2]))
    return out


def pair_alpha(px, py, mean2d, conic, opacity):
    """v = o exp(-q/2) and the float32 error bound rel (relative) of the compositing's error
    model for n arbitrary (pixel centre, record) pairs: px, py (n,), mean2d (n,2), conic (n,3),
    opacity (n,).  Returns (v, rel)."""
    lib = _load()
    px = np.ascontiguousarray(px, np.float64)
    py = np.ascontiguousarray(py, np.float64)
    m = np.ascontiguousarray(mean2d, np.float64)
    c = np.ascontiguousarray(conic, np.float64)
    o = np.ascontiguousarray(opacity, np.float64)
    n = px.size
    v = np.zeros(n)
    rel = np.zeros(n)
    lib.orc_pair_alpha(ctypes.c_int64(n), _p(px), _p(py), _p(m), _p(c), _p(o), _p(v), _p(rel))
    return v, rel


def raster_bruteforce(width: int, height: int, order: np.ndarray, records: dict, settings) -> dict:
    """All slots composited at every pixel in the given global order (no tiles)."""
    lib = _load()
    image = np.zeros((3, height, width))
    T = np.zeros((height, width))
    nc = np.zeros((height, width), np.int32)
    order = np.ascontiguousarray(order, np.int32)
    pp = _params(settings)
    m, c, o, col = _rec(records)
    lib.orc_raster_bruteforce(ctypes.c_int32(width), ctypes.c_int32(height), _p(order), ctypes.c_int32(order.size),
                              _p(m), _p(c), _p(o), _p(col), ctypes.byref(pp), _p(image), _p(T), _p(nc))
    return dict(image=image, T_final=T, n_contrib=nc)


# ---------------------------------------------------------------------------------------
# One iteration over all views
# ---------------------------------------------------------------------------------------
def iteration(scene, settings, loss_scale: float = 1.0, views=None, backward: bool = True) -> list:
    """project -> compact -> bin (-> cap) -> forward -> loss gradient -> backward, per view.

    The views of a batch are independent renders (Grendel, arXiv 2406.18533, English
    abstract: batched training over several views); per-view 2D gradients are not summed."""
    out = []
    views = range(len(scene.cameras)) if views is None else views
    for v in views:
        cam = scene.cameras[v]
        proj = project(scene, cam, settings)
        rec = compact(proj)
        dbits = depth_bits(rec["depth"])
        bins = bin_tiles(rec["rect"], rec["n_tiles"], dbits, cam.tiles_x, cam.tiles_y)
        ranges, vals = bins["ranges"], bins["vals"]
        if settings.tile_cap > 0:
            score = cap_score(rec["conic"].astype(np.float32), rec["opacity"].astype(np.float32))
            capped = cap_tiles(ranges, vals, score, dbits, settings.tile_cap)
            ranges, vals = capped["ranges"], capped["vals"]
            bins["capped"] = capped
        fwd = raster_forward(cam.width, cam.height, ranges, vals, rec, settings)
        res = dict(view=v, proj=proj, rec=rec, bins=bins, fwd=fwd)
        if backward:
            if scene.loss == "l1":
                g, dg = loss_grad_l1(fwd["image"], scene.target[v], loss_scale, fwd["err_C"])
            else:
                g, dg = scene.dldc[v].astype(np.float64), None
            res["dldc"] = g
            res["bwd"] = raster_backward(cam.width, cam.height, ranges, vals, rec, settings, g, dg=dg)
        out.append(res)
    return out


def grad_records(vis_count, d_mean2d, d_conic, d_opacity, d_color) -> list:
    """The nine-component 2D gradient record of every visible slot, per view:
    (mean2d x, y, conic A, B, C, opacity, colour r, g, b).  Inputs are [V][capacity][...]."""
    out = []
    for v, n in enumerate(vis_count):
        n = int(n)
        out.append(np.concatenate([np.asarray(d_mean2d[v][:n]).reshape(n, 2), np.asarray(d_conic[v][:n]).reshape(n, 3),
                                   np.asarray(d_opacity[v][:n]).reshape(n, 1), np.asarray(d_color[v][:n]).reshape(n, 3)],
                                  axis=1))
    return out


def grad_encode(vis_count, vis_ids, records_per_view: list) -> dict:
    """Sparse encoding of partial gradients (ByteSplat, English abstract: zero partial gradients
    are left out of the exchange, and an encoder compacts the remaining records).  Per view in
    slot order, a record is kept when any component differs from zero (NaN != 0 holds, so a NaN is
    kept; -0 == 0, so -0 is dropped); it carries the slot's Gaussian index.  Returns keys,
    records (K, 9) and view_offset (V + 1).
    Parity: pinned by the round trip to the dense scatter and by counts from an explicit loop."""
    keys, recs, off = [], [], [0]
    for v, R in enumerate(records_per_view):
        R = np.asarray(R)
        keep = np.any(R != 0, axis=1)
        keys.append(np.asarray(vis_ids[v][:R.shape[0]])[keep])
        recs.append(R[keep])
        off.append(off[-1] + int(keep.sum()))
    return dict(keys=np.concatenate(keys) if keys else np.zeros(0, np.int32),
                records=np.concatenate(recs) if recs else np.zeros((0, 9)), view_offset=np.array(off, np.int64))


def grad_decode(view_offset, keys, records, owner: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Aggregation on the owner (ByteSplat, English abstract: the decoder adds the received
    gradients directly into the owner's arrays): owner[v, keys[k]] += records[k] for every record
    k of view v, keys outside [0, n_owner) skipped, in `dtype` arithmetic.  owner is [V][n_owner][9].
    Parity: pinned by the round trip to the dense scatter and by stream accumulation."""
    out = np.array(owner, dtype=dtype, copy=True)
    n_owner = out.shape[1]
    for v in range(out.shape[0]):
        for k in range(int(view_offset[v]), int(view_offset[v + 1])):
            g = int(keys[k])
            if 0 <= g < n_owner:
                out[v, g] = (out[v, g] + np.asarray(records[k], dtype=dtype)).astype(dtype)
    return out


def compose(colors: list, t_finals: list, bg) -> tuple:
    """Global composition of pixel-level partial renders (Splaxel, English abstract: each GPU
    renders its local subset and partial pixel values are composed into the image).  Partials
    are (premultiplied colour C [V][3][H][W] drawn on black, final transmittance T [V][H][W]) in
    front-to-back order; front to back, C += T_acc C_i and T_acc *= T_i, and the background is
    added once: image = C + T_acc bg.  Float64.  Returns (image, T_acc).
    Parity: pinned by the exactness of composing depth-separated subsets against compositing
    their union (t_min = 0), identity of a transparent partial, and associativity."""
    C = np.zeros(np.shape(colors[0]), np.float64)
    T = np.ones(np.shape(t_finals[0]), np.float64)
    for c, t in zip(colors, t_finals):
        C = C + T[:, None] * np.asarray(c, np.float64)
        T = T * np.asarray(t, np.float64)
    bgv = np.asarray(bg, np.float64).reshape(1, 3, 1, 1)
    return C + T[:, None] * bgv, T


def adam(params: list, grads_per_step: list, lrs: list, beta1: float, beta2: float, eps: float) -> tuple:
    """Textbook Adam (the optimizer whose deferred update GS-Scale's English abstract describes as
    skipping the memory accesses of Gaussians with zero gradients; the deferred form must equal
    this one): for t = 1, 2, ..., per component, m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
    p -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).  Float64.  params: list of arrays
    (one per group); grads_per_step: list over steps of lists of arrays.  Returns (params, m, v).
    Parity: pinned against torch.optim.Adam (float64, CPU), the first-step closed form
    p - lr g / (|g| + eps) and the zero-gradient decay of the moments."""
    p = [np.array(x, np.float64, copy=True) for x in params]
    m = [np.zeros_like(x) for x in p]
    v = [np.zeros_like(x) for x in p]
    for t, grads in enumerate(grads_per_step, start=1):
        bc1, bc2 = 1.0 - beta1 ** t, 1.0 - beta2 ** t
        for k, g in enumerate(grads):
            g = np.asarray(g, np.float64)
            m[k] = beta1 * m[k] + (1.0 - beta1) * g
            v[k] = beta2 * v[k] + (1.0 - beta2) * g * g
            p[k] = p[k] - lrs[k] * ((m[k] / bc1) / (np.sqrt(v[k] / bc2) + eps))
    return p, m, v
