"""Pins of the oracle's projection backward (chain rule from the 2D gradients of mean2d, conic,
opacity and colour to the 3D parameters: means, log-scales, raw quaternions, opacity logits, SH).

The pages name training of the splats (ByteSplat, English abstract) but write out no
derivative; the oracle's backward is the chain rule of its own projection.  It is pinned here
against things other than itself:
* central finite differences of the double-precision projection, for every parameter
  component, on posed cameras with fx != fy, anisotropic rotated Gaussians and SH degree 3;
* the SH basis gradient against finite differences of the SH basis (itself pinned to scipy);
* invariances: an isotropic Gaussian's covariance does not depend on its rotation (zero
  quaternion gradient); the projection does not depend on the quaternion's norm (gradient
  orthogonal to the quaternion); per-view calls add up.
"""
import numpy as np
import pytest

from differentiable_raster_amd import scenes
from helpers import pinhole, scene_from


def _rot(ax, ang):
    c, s = np.cos(ang), np.sin(ang)
    if ax == 0:
        return np.array([[1, 0, 0], [0, c, -s], [0, s, c]])
    if ax == 1:
        return np.array([[c, 0, s], [0, 1, 0], [-s, 0, c]])
    return np.array([[c, -s, 0], [s, c, 0], [0, 0, 1]])


def _posed_cameras():
    R1 = (_rot(1, 0.3) @ _rot(0, -0.2)).astype(np.float32)
    t1 = np.array([0.3, -0.2, 0.5], np.float32)
    return [pinhole(96, 64, f=80.0, fy=70.0, cx=47.5, cy=33.0),
            pinhole(96, 64, f=90.0, fy=101.0, cx=50.0, cy=30.0, R=R1, t=t1)]


def _scene(n=300, seed=3, deg=3):
    sc = scenes.random_scene(n, 96, 64, seed, views=1, sh_degree=deg, z_range=(1.5, 5.0), xy_extent=1.2,
                             log_scale_mean=-2.5, log_scale_std=0.6)
    sc.cameras = _posed_cameras()
    return sc


def _loss_terms(oracle, params, cam, st, g):
    """Per-Gaussian contributions of L = sum over visible Gaussians of <g, projected outputs>."""
    o = oracle.project_f64(params, cam, st)
    terms = ((g["mean2d"] * o["mean2d"]).sum(1) + (g["conic"] * o["conic"]).sum(1) + g["opacity"] * o["opacity"]
             + (g["color"] * o["color"]).sum(1))
    return np.where(o["visible"] == 1, terms, 0.0), o["visible"]


def _random_g(rng, n):
    return dict(mean2d=rng.standard_normal((n, 2)), conic=rng.standard_normal((n, 3)) * 0.1,
                opacity=rng.standard_normal(n), color=rng.standard_normal((n, 3)))


KEYS = [("means", "d_means"), ("log_scales", "d_log_scales"), ("quats", "d_quats"),
        ("opacity_logits", "d_opacity_logits"), ("sh", "d_sh")]


@pytest.mark.parametrize("view", [0, 1])
def test_projection_backward_matches_finite_differences(oracle_mod, view):
    oracle = oracle_mod
    sc = _scene()
    st = sc.settings()
    cam = sc.cameras[view]
    params = oracle.scene_params_f64(sc)
    n = sc.n
    rng = np.random.default_rng(11 + view)
    g = _random_g(rng, n)
    base = oracle.project_f64(params, cam, st)
    vis = base["visible"]
    assert vis.sum() > 100
    acc = oracle.project_backward(params, cam, st, vis, g["mean2d"], g["conic"], g["opacity"], g["color"])
    ok = (vis == 1) & (acc["flag"] == 0)
    checked = 0
    for pk, gk in KEYS:
        arr = params[pk]
        rows = arr.shape[0] if arr.ndim == 2 else 1
        for r in range(rows):
            h = 1e-6 * max(1.0, float(np.abs(arr[r]).max()))
            plus = {k: v.copy() for k, v in params.items()}
            minus = {k: v.copy() for k, v in params.items()}
            if arr.ndim == 2:
                plus[pk][r] += h
                minus[pk][r] -= h
            else:
                plus[pk] += h
                minus[pk] -= h
            lp, vp = _loss_terms(oracle, plus, cam, st, g)
            lm, vm = _loss_terms(oracle, minus, cam, st, g)
            fd = (lp - lm) / (2 * h)
            an = acc[gk][r] if arr.ndim == 2 else acc[gk]
            sel = ok & (vp == 1) & (vm == 1)
            err = np.abs(an[sel] - fd[sel])
            bound = 1e-6 * np.abs(fd[sel]) + 1e-6 * max(1.0, np.abs(fd[sel]).max())
            assert (err <= bound).all(), (pk, r, float(err.max()), float(np.abs(fd[sel]).max()))
            checked += int(sel.sum())
    assert checked > 59 * 100


def test_sh_basis_grad_matches_finite_differences(oracle_mod):
    oracle = oracle_mod
    rng = np.random.default_rng(5)
    pts = rng.standard_normal((50, 3))
    pts[:25] /= np.linalg.norm(pts[:25], axis=1, keepdims=True)
    for deg in range(4):
        dY = oracle.sh_basis_grad(deg, pts)
        h = 1e-6
        for m in range(3):
            e = np.zeros(3)
            e[m] = h
            fd = (oracle.sh_basis(deg, pts + e) - oracle.sh_basis(deg, pts - e)) / (2 * h)
            assert np.allclose(dY[:, :, m], fd, rtol=1e-7, atol=1e-8)


def test_isotropic_gaussian_has_no_rotation_gradient(oracle_mod):
    oracle = oracle_mod
    cams = _posed_cameras()
    rng = np.random.default_rng(2)
    n = 40
    means = np.column_stack([rng.uniform(-0.8, 0.8, n), rng.uniform(-0.5, 0.5, n), rng.uniform(2, 4, n)])
    ls = np.repeat(rng.uniform(-3, -2, (n, 1)), 3, axis=1)
    quats = rng.standard_normal((n, 4))
    sc = scene_from(means, ls, quats, rng.standard_normal(n), rng.uniform(0.2, 0.8, (n, 3)), cams)
    st = sc.settings()
    params = oracle.scene_params_f64(sc)
    g = _random_g(rng, n)
    for cam in cams:
        vis = oracle.project_f64(params, cam, st)["visible"]
        assert vis.sum() > 10
        acc = oracle.project_backward(params, cam, st, vis, g["mean2d"], g["conic"], g["opacity"], g["color"])
        # the covariance is s^2 I whatever the rotation: every quaternion gradient vanishes
        assert np.abs(acc["d_quats"]).max() <= 1e-9 * max(1.0, np.abs(acc["d_log_scales"]).max())
        assert np.abs(acc["d_log_scales"][:, vis == 1]).max() > 1e-3


def test_quaternion_gradient_is_orthogonal_and_views_add(oracle_mod):
    oracle = oracle_mod
    sc = _scene(n=200, seed=9)
    st = sc.settings()
    params = oracle.scene_params_f64(sc)
    # scale the raw quaternions: the projection, and so L, is unchanged, so d/dq . q = 0
    params["quats"] = params["quats"] * np.linspace(0.5, 2.0, sc.n)[None, :]
    rng = np.random.default_rng(4)
    gs = [_random_g(rng, sc.n) for _ in sc.cameras]
    acc = None
    single = []
    for cam, g in zip(sc.cameras, gs):
        vis = oracle.project_f64(params, cam, st)["visible"]
        acc = oracle.project_backward(params, cam, st, vis, g["mean2d"], g["conic"], g["opacity"], g["color"], acc)
        single.append(oracle.project_backward(params, cam, st, vis, g["mean2d"], g["conic"], g["opacity"],
                                              g["color"]))
    radial = (acc["d_quats"] * params["quats"]).sum(0)
    assert np.abs(radial).max() <= 1e-10 * max(1.0, np.abs(acc["d_quats"]).max())
    for k in ("d_means", "d_log_scales", "d_quats", "d_opacity_logits", "d_sh"):
        assert np.allclose(acc[k], single[0][k] + single[1][k], rtol=1e-13, atol=1e-15)


def test_colour_and_opacity_terms_closed_form(oracle_mod):
    """SH coefficient gradients are g * Y_k(dir) (g for the DC) while the channel is unclamped,
    zero when clamped; the opacity-logit gradient is g_o * o (1 - o)."""
    oracle = oracle_mod
    cam = pinhole(64, 64, f=60.0)
    n = 3
    means = [[0.0, 0.0, 3.0], [0.2, -0.1, 2.5], [-0.3, 0.2, 4.0]]
    dc = [[0.5, 0.3, 0.2], [0.4, -2.0, 0.6], [0.1, 0.2, 0.3]]  # second Gaussian: green clamped at 0
    rest = np.random.default_rng(0).standard_normal((n, 45)) * 0.05
    sc = scene_from(means, [[-2.5] * 3] * n, [[1, 0, 0, 0]] * n, [0.3, -0.7, 1.1], dc, [cam], sh_rest=rest,
                    sh_degree=3)
    st = sc.settings()
    params = oracle.scene_params_f64(sc)
    vis = oracle.project_f64(params, cam, st)["visible"]
    assert vis.tolist() == [1, 1, 1]
    g_col = np.array([[1.0, -2.0, 0.5], [0.7, 0.9, -1.3], [0.0, 1.0, 2.0]])
    g_op = np.array([0.4, -1.5, 2.0])
    z = np.zeros((n, 2))
    acc = oracle.project_backward(params, cam, st, vis, z, np.zeros((n, 3)), g_op, g_col)
    o = 1.0 / (1.0 + np.exp(-params["opacity_logits"]))
    assert np.allclose(acc["d_opacity_logits"], g_op * o * (1 - o), rtol=1e-14)
    mu = params["means"].T
    d = mu - np.asarray(cam.campos, np.float64)[None, :]
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    Y = oracle.sh_basis(3, d)
    for i in range(n):
        for ch in range(3):
            v = params["sh"][ch, i] + sum(params["sh"][k * 3 + ch, i] * Y[i, k] for k in range(1, 16))
            live = v > 0
            assert acc["d_sh"][ch, i] == pytest.approx(g_col[i, ch] if live else 0.0, abs=1e-15)
            for k in range(1, 16):
                want = g_col[i, ch] * Y[i, k] if live else 0.0
                assert acc["d_sh"][k * 3 + ch, i] == pytest.approx(want, rel=1e-13, abs=1e-15)
    # the clamped channel really is the second Gaussian's green
    v_g = params["sh"][1, 1] + sum(params["sh"][k * 3 + 1, 1] * Y[1, k] for k in range(1, 16))
    assert v_g < 0


def _chain_float32(params, cam, vis, g):
    """The projection backward for one view evaluated in plain numpy float32 (no fused
    multiply-adds), vectorized over Gaussians: a float32 evaluation against which the oracle's
    rounding-error bound is checked."""
    f = np.float32
    n = params["means"].shape[1]
    P = {k: np.asarray(v, f) for k, v in params.items()}
    mu = P["means"]
    s = np.exp(P["log_scales"])
    qr = P["quats"]
    qn = np.sqrt((qr * qr).sum(0, dtype=f)).astype(f)
    q = qr / qn
    w, x, y, z = q
    one, two = f(1), f(2)
    Rq = np.stack([one - two * (y * y + z * z), two * (x * y - w * z), two * (x * z + w * y),
                   two * (x * y + w * z), one - two * (x * x + z * z), two * (y * z - w * x),
                   two * (x * z - w * y), two * (y * z + w * x), one - two * (x * x + y * y)]).reshape(3, 3, n)
    M = Rq * s[None, :, :]
    Sig = np.einsum("akn,bkn->abn", M, M).astype(f)
    W = np.asarray(cam.R, f).reshape(3, 3)
    tc = (np.einsum("rk,kn->rn", W, mu) + np.asarray(cam.t, f)[:, None]).astype(f)
    fx, fy = f(cam.fx), f(cam.fy)
    iz = one / tc[2]
    J = np.zeros((2, 3, n), f)
    J[0, 0] = fx * iz
    J[0, 2] = -fx * tc[0] * iz * iz
    J[1, 1] = fy * iz
    J[1, 2] = -fy * tc[1] * iz * iz
    T = np.einsum("rkn,kc->rcn", J, W).astype(f)
    U = np.einsum("abn,bn->an", Sig, T[0]).astype(f)
    Vv = np.einsum("abn,bn->an", Sig, T[1]).astype(f)
    eps = f(0.3)
    a = (T[0] * U).sum(0, dtype=f) + eps
    b = (T[1] * U).sum(0, dtype=f)
    c = (T[1] * Vv).sum(0, dtype=f) + eps
    det = a * c - b * b
    idet = one / det
    A, B, C = c * idet, -b * idet, a * idet
    gA, gB, gC = [np.asarray(g["conic"][:, k], f) for k in range(3)]
    ga = -(A * A * gA + A * B * gB + B * B * gC)
    gb = -(two * A * B * gA + (A * C + B * B) * gB + two * B * C * gC)
    gc = -(B * B * gA + B * C * gB + C * C * gC)
    gT0 = two * ga * U + gb * Vv
    gT1 = gb * U + two * gc * Vv
    Gs = (two * ga * T[0][:, None] * T[0][None] + gb * (T[0][:, None] * T[1][None] + T[1][:, None] * T[0][None])
          + two * gc * T[1][:, None] * T[1][None]).astype(f)
    gJ0 = np.einsum("cn,kc->kn", gT0, W).astype(f)
    gJ1 = np.einsum("cn,kc->kn", gT1, W).astype(f)
    gm = np.asarray(g["mean2d"], f).T
    iz2 = iz * iz
    gt = np.stack([gm[0] * fx * iz - gJ0[2] * fx * iz2,
                   gm[1] * fy * iz - gJ1[2] * fy * iz2,
                   -gm[0] * fx * tc[0] * iz2 - gm[1] * fy * tc[1] * iz2 - gJ0[0] * fx * iz2
                   + two * gJ0[2] * fx * tc[0] * iz2 * iz - gJ1[1] * fy * iz2 + two * gJ1[2] * fy * tc[1] * iz2 * iz])
    gmu = np.einsum("rk,rn->kn", W, gt).astype(f)
    out = {}
    sk2 = s * s
    wv = np.einsum("uvn,vkn->ukn", Gs, Rq).astype(f)  # Gs times column k of Rq
    out["d_log_scales"] = sk2 * (Rq * wv).sum(0, dtype=f)
    gR = (wv * sk2[None]).astype(f)
    gq = two * np.stack([
        -z * gR[0, 1] + y * gR[0, 2] + z * gR[1, 0] - x * gR[1, 2] - y * gR[2, 0] + x * gR[2, 1],
        y * gR[0, 1] + z * gR[0, 2] + y * gR[1, 0] - two * x * gR[1, 1] - w * gR[1, 2] + z * gR[2, 0]
        + w * gR[2, 1] - two * x * gR[2, 2],
        -two * y * gR[0, 0] + x * gR[0, 1] + w * gR[0, 2] + x * gR[1, 0] + z * gR[1, 2] - w * gR[2, 0]
        + z * gR[2, 1] - two * y * gR[2, 2],
        -two * z * gR[0, 0] - w * gR[0, 1] + x * gR[0, 2] + w * gR[1, 0] - two * z * gR[1, 1] + y * gR[1, 2]
        + x * gR[2, 0] + y * gR[2, 1]])
    qd = (gq * q).sum(0, dtype=f)
    out["d_quats"] = (gq - q * qd) / qn
    o = one / (one + np.exp(-P["opacity_logits"]))
    out["d_opacity_logits"] = np.asarray(g["opacity"], f) * o * (one - o)
    dv = mu - np.asarray(cam.campos, f)[:, None]
    dn = np.sqrt((dv * dv).sum(0, dtype=f))
    d = dv / dn
    deg = int(round(np.sqrt(P["sh"].shape[0] // 3))) - 1
    import oracle as orc
    Y = orc.sh_basis(deg, d.T.astype(np.float64)).astype(f)
    dY = orc.sh_basis_grad(deg, d.T.astype(np.float64)).astype(f)
    nk = (deg + 1) ** 2
    dsh = np.zeros((3 * nk, n), f)
    gdir = np.zeros((3, n), f)
    for ch in range(3):
        val = P["sh"][ch] + sum(P["sh"][k * 3 + ch] * Y[:, k] for k in range(1, nk))
        live = (val > 0).astype(f)
        gch = np.asarray(g["color"][:, ch], f) * live
        dsh[ch] = gch
        for k in range(1, nk):
            dsh[k * 3 + ch] = gch * Y[:, k]
            gdir += (gch * P["sh"][k * 3 + ch])[None] * dY[:, k, :].T
    r = (gdir * d).sum(0, dtype=f)
    gmu = gmu + (gdir - d * r) / dn
    out["d_means"] = gmu
    out["d_sh"] = dsh
    return {k: np.where(vis[None] == 1, v, 0) if v.ndim == 2 else np.where(vis == 1, v, 0) for k, v in out.items()}


@pytest.mark.parametrize("view", [0, 1])
def test_error_bound_covers_a_float32_evaluation(oracle_mod, view):
    """The oracle's first-order float32 error bound of the projection backward covers the
    difference between a plain float32 evaluation of the chain and the double-precision oracle,
    and is not vacuous (far below the values for most components)."""
    oracle = oracle_mod
    sc = _scene(n=2000, seed=21)
    st = sc.settings()
    cam = sc.cameras[view]
    params = oracle.scene_params_f64(sc)
    rng = np.random.default_rng(13 + view)
    # float32 inputs, as the kernel receives them (the bound models the arithmetic, not the inputs)
    g = {k: v.astype(np.float32).astype(np.float64) for k, v in _random_g(rng, sc.n).items()}
    vis = oracle.project_f64(params, cam, st)["visible"]
    acc = oracle.project_backward(params, cam, st, vis, g["mean2d"], g["conic"], g["opacity"], g["color"],
                                  error_bound=True)
    f32 = _chain_float32(params, cam, vis, g)
    use = (vis == 1) & (acc["flag"] == 0)
    for k in ("d_means", "d_log_scales", "d_quats", "d_opacity_logits", "d_sh"):
        o = acc[k][..., use]
        e = acc["e" + k[1:]][..., use]
        err = np.abs(f32[k][..., use].astype(np.float64) - o)
        ratio = err / (2.0 * e + 1e-300)
        assert (err <= 2.0 * e + 1e-30).all(), (k, float(ratio.max()))
        # not vacuous: the bound's median relative size (larger where the chain cancels by
        # construction: the scale and rotation gradients sum terms of both signs)
        rel_bound = e / (np.abs(o) + 1e-30)
        limit = {"d_log_scales": 1e-3, "d_quats": 1e-2}.get(k, 1e-4)
        assert np.median(rel_bound) < limit, (k, float(np.median(rel_bound)))
