"""Pins of the oracle's float32 error model of the compositing (the tolerance model the parity
comparisons use): evaluations of the same compositing in float32, emulated in NumPy, must stay
within the oracle's bounds, and the bounds must not be vacuous.

The emulation rounds every +, -, x and fused multiply-add correctly (IEEE round to nearest) and
takes every exponential, logarithm and reciprocal as faithful: at random the float32 neighbour
below or above the exact value (error under one ulp), a fresh choice per evaluation.  Two
evaluation orders are emulated:
  * the definition's: q = A dx^2 + 2B dx dy + C dy^2 term by term, exp(-q/2), times o;
  * base 2: p = a dx^2 + b dx dy + c dy^2 + log2 o with pre-scaled coefficients, added by fused
    multiply-adds, then exp2(p), and the alpha_min test taken on p against log2(alpha_min).
Compositing: alpha = min(alpha_max, v), 1 - alpha, T (1 - alpha), the colour sum; the backward
recovers T_j from T_final by multiplying with a faithful reciprocal of 1 - alpha and carries the
colour behind as the running sum GB, as the oracle's backward describes.

What is checked:
  * per pair: |v32 - v| <= rel v (the alpha budget), for o over [alpha_min, 1] and q over the
    whole alpha_min box; every alpha_min decision float32 takes differently lies inside the
    flagged band;
  * per pixel: pixels without a flagged decision reach the same n_contrib, colour within err_C
    and T_final within err_T T_final; a pixel with flagged decisions equals one of the oracle's
    alternatives (the same decisions taken the other way) within the same bounds;
  * per slot: the float32 gradients (contributions summed over pixels in a random order) lie
    within the summed contribution bounds err plus m u mag for a sum of m contributions, plus
    the widening of the flagged pixels;
  * on the workload scene of 4 096 Gaussians, a random scene, and stacks of near-opaque
    splats (alpha 0.95 to 0.99) where 1 / (1 - alpha) amplifies every rounding of alpha.
"""
import numpy as np
import pytest

from differentiable_raster_amd import scenes

U = 2.0 ** -24
F = np.float32
LOG2E = F(1.4426950408889634)
LN2 = F(0.6931471805599453)


class Float32:
    """Float32 arithmetic with correctly rounded basic operations and faithful transcendentals."""

    def __init__(self, seed):
        self.rng = np.random.default_rng(seed)

    def faithful(self, x64):
        x64 = np.asarray(x64, np.float64)
        f = x64.astype(F)
        f64 = f.astype(np.float64)
        up = np.nextafter(f, F(np.inf))
        dn = np.nextafter(f, F(-np.inf))
        lo = np.where(f64 <= x64, f, dn)
        hi = np.where(f64 >= x64, f, up)
        return np.where(self.rng.random(x64.shape) < 0.5, lo, hi).astype(F)

    @staticmethod
    def fma(a, b, c):
        # a*b is exact in float64; one more rounding to 53 bits before the final one is far
        # below the bounds under test
        return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(F)

    def exp(self, x):
        return self.faithful(np.exp(np.asarray(x, np.float64)))

    def exp2(self, x):
        return self.faithful(np.exp2(np.asarray(x, np.float64)))

    def log2(self, x):
        return self.faithful(np.log2(np.asarray(x, np.float64)))

    def rcp(self, x):
        return self.faithful(1.0 / np.asarray(x, np.float64))


def pair_v32(ar: Float32, order, px, py, mx, my, A, B, C, o):
    """v = o exp(-q/2) in float32; all inputs float32 arrays.  Returns (v32, p2 or None)."""
    dx = px - mx
    dy = py - my
    if order == "definition":
        t1 = (A * dx) * dx
        t2 = ((F(2) * B) * dx) * dy
        t3 = (C * dy) * dy
        q = (t1 + t2) + t3
        return o * ar.exp(F(-0.5) * q), None
    ca = F(-0.5) * LOG2E
    a, b, c = ca * A, -LOG2E * B, ca * C
    l = ar.log2(o)
    s1 = ar.fma(c * dy, dy, l)
    s2 = ar.fma(b * dx, dy, s1)
    p2 = ar.fma(a * dx, dx, s2)
    return ar.exp2(p2), p2


# ------------------------------------------------------------------------------------------
# per pair
# ------------------------------------------------------------------------------------------
def random_pairs(rng, n):
    """Records and pixel centres over the whole alpha_min box: opacity log-uniform in
    [alpha_min, 1], 2D covariances with eigenvalues 0.3 .. 1e4 px^2 at random angles, centres
    anywhere on a 4K image, pixels at random Mahalanobis radii inside the box."""
    amin = 1.0 / 255.0
    o = np.exp(rng.uniform(np.log(amin * 1.0001), 0.0, n)).astype(F)
    l1 = np.exp(rng.uniform(np.log(0.3), np.log(1e4), n))
    l2 = np.exp(rng.uniform(np.log(0.3), np.log(1e4), n))
    th = rng.uniform(0, np.pi, n)
    c, s = np.cos(th), np.sin(th)
    sxx = c * c * l1 + s * s * l2
    syy = s * s * l1 + c * c * l2
    sxy = c * s * (l1 - l2)
    det = sxx * syy - sxy * sxy
    A = (syy / det).astype(F)
    B = (-sxy / det).astype(F)
    C = (sxx / det).astype(F)
    mx = rng.uniform(0, 3840, n).astype(F)
    my = rng.uniform(0, 2160, n).astype(F)
    # a point at Mahalanobis radius r (q = r^2) up to slightly past the alpha_min contour
    qmax = 2.0 * np.log(o.astype(np.float64) / amin)
    r = np.sqrt(rng.uniform(0, 1.05, n) * qmax)
    phi = rng.uniform(0, 2 * np.pi, n)
    L = np.linalg.cholesky(np.stack([np.stack([sxx, sxy], -1), np.stack([sxy, syy], -1)], -2))
    z = np.stack([r * np.cos(phi), r * np.sin(phi)], -1)
    off = np.einsum("nij,nj->ni", L, z)
    px = (np.floor(mx + off[:, 0]) + 0.5).astype(F)
    py = (np.floor(my + off[:, 1]) + 0.5).astype(F)
    return px, py, mx, my, A, B, C, o


@pytest.mark.parametrize("order", ["definition", "base2"])
def test_alpha_error_bound_covers_float32(oracle_mod, order):
    rng = np.random.default_rng(11)
    amin = F(1.0 / 255.0)
    worst = 0.0
    rels = []
    for seed in range(4):
        px, py, mx, my, A, B, C, o = random_pairs(rng, 200_000)
        v, rel = oracle_mod.pair_alpha(px, py, np.stack([mx, my], 1), np.stack([A, B, C], 1), o)
        ar = Float32(100 + seed)
        v32, p2 = pair_v32(ar, order, px, py, mx, my, A, B, C, o)
        err = np.abs(v32.astype(np.float64) - v)
        ok = err <= rel * v
        assert ok.all(), f"{int((~ok).sum())} pairs outside the bound, worst ratio {float((err / (rel * v)).max())}"
        worst = max(worst, float((err / (rel * v)).max()))
        rels.append(rel)
        # decisions: float32 takes alpha >= alpha_min differently only inside the flagged band
        if order == "base2":
            dec32 = p2 >= ar.log2(np.full(px.shape, amin))
        else:
            dec32 = v32 >= amin
        dec64 = v >= float(amin)
        thr = 2.0 * U * abs(np.log(float(amin)))
        flipped = dec32 != dec64
        band = np.abs(v - float(amin)) <= (rel + thr) * float(amin)
        assert not (flipped & ~band).any(), "an alpha_min decision flipped outside the flagged band"
    rels = np.concatenate(rels)
    print(f"[error model] {order}: worst |v32 - v| / (rel v) = {worst:.3f}; rel median {np.median(rels) / U:.1f} u, "
          f"max {rels.max() / U:.1f} u")
    # not vacuous: the bound is within a factor 8 of the worst error seen, and a few dozen ulp
    assert worst >= 0.125
    assert np.median(rels) <= 48 * U


# ------------------------------------------------------------------------------------------
# per pixel and per slot
# ------------------------------------------------------------------------------------------
def f32_records(rec64: dict) -> dict:
    """Round records to float32 (the values a float32 rasterizer reads) and widen them back."""
    return {k: np.asarray(rec64[k], F).astype(np.float64) for k in ("mean2d", "conic", "opacity", "color")}


def scene_records(oracle_mod, sc, view=0):
    st = sc.settings()
    cam = sc.cameras[view]
    proj = oracle_mod.project(sc, cam, st)
    rec = oracle_mod.compact(proj)
    recs = f32_records(rec)
    depth = np.asarray(rec["depth"], F)
    b = oracle_mod.bin_tiles(rec["rect"], rec["n_tiles"], depth.view(np.uint32), cam.tiles_x, cam.tiles_y)
    return cam.width, cam.height, b["ranges"], b["vals"], recs, st


def opaque_stack_records(rng, W=48, H=48, n=240):
    """Near-opaque splats (opacity 0.95 to 0.995, so alpha reaches the 0.99 clamp at some
    centres) stacked over a small image: every pixel meets several alpha 0.95..0.99 entries
    in a row, and T reaches t_min.  Records are given directly in screen space (sorted by a
    random depth), one list for all tiles."""
    mean = np.stack([rng.uniform(0, W, n), rng.uniform(0, H, n)], 1)
    l1 = np.exp(rng.uniform(np.log(4.0), np.log(60.0), n))
    l2 = np.exp(rng.uniform(np.log(4.0), np.log(60.0), n))
    th = rng.uniform(0, np.pi, n)
    c, s = np.cos(th), np.sin(th)
    sxx, syy, sxy = c * c * l1 + s * s * l2 + 0.3, s * s * l1 + c * c * l2 + 0.3, c * s * (l1 - l2)
    det = sxx * syy - sxy * sxy
    conic = np.stack([syy / det, -sxy / det, sxx / det], 1)
    opacity = rng.uniform(0.95, 0.995, n)
    color = rng.uniform(0, 1, (n, 3))
    recs = f32_records(dict(mean2d=mean, conic=conic, opacity=opacity, color=color))
    tiles = ((W + 15) // 16) * ((H + 15) // 16)
    vals = np.concatenate([np.arange(n, dtype=np.int32)] * tiles)
    ranges = np.stack([np.arange(tiles) * n, np.arange(1, tiles + 1) * n], 1).astype(np.int32)
    return W, H, ranges, vals, recs


def emulate(oracle_mod, W, H, ranges, vals, recs, st, order, seed, dldc):
    """Float32 forward and backward of every pixel over its tile's list.  Returns image (3,H,W),
    T (H,W), n_contrib (H,W) and per slot the gradient sums (S,9) plus the number of
    contributions summed into each slot."""
    ar = Float32(seed)
    S = recs["opacity"].shape[0]
    m32 = recs["mean2d"].astype(F)
    c32 = recs["conic"].astype(F)
    o32 = recs["opacity"].astype(F)
    col32 = recs["color"].astype(F)
    amin, amax, tmin = F(st.alpha_min), F(st.alpha_max), F(st.t_min)
    bg = np.asarray(st.bg, F)
    l2amin = ar.log2(np.asarray([amin]))[0]
    image = np.zeros((3, H, W), F)
    Tout = np.zeros((H, W), F)
    ncout = np.zeros((H, W), np.int32)
    contrib = []  # (slot, pixel id, 9 values) per blended pair, gathered per tile
    tx_n = (W + 15) // 16
    for t in range(ranges.shape[0]):
        s0, s1 = int(ranges[t, 0]), int(ranges[t, 1])
        tx, ty = t % tx_n, t // tx_n
        ys, xs = np.mgrid[ty * 16:min(H, ty * 16 + 16), tx * 16:min(W, tx * 16 + 16)]
        xs, ys = xs.ravel(), ys.ravel()
        P = xs.size
        if P == 0:
            continue
        pxc = (xs + 0.5).astype(F)
        pyc = (ys + 0.5).astype(F)
        lst = vals[s0:s1]
        n = lst.size
        T = np.ones(P, F)
        Cc = np.zeros((3, P), F)
        nc = np.zeros(P, np.int32)
        done = np.zeros(P, bool)
        blended = np.zeros((n, P), bool)
        vs = np.zeros((n, P), F)
        als = np.zeros((n, P), F)
        for j, s in enumerate(lst):
            if done.all():
                break
            mx, my = np.full(P, m32[s, 0]), np.full(P, m32[s, 1])
            A, B, C, o = (np.full(P, x) for x in (c32[s, 0], c32[s, 1], c32[s, 2], o32[s]))
            v, p2 = pair_v32(ar, order, pxc, pyc, mx, my, A, B, C, o)
            hit = (p2 >= l2amin) if order == "base2" else (np.minimum(v, amax) >= amin)
            alpha = np.minimum(v, amax)
            oma = F(1) - alpha
            Tn = T * oma
            blend = ~done & hit & ~(Tn < tmin)
            stop = ~done & hit & (Tn < tmin)
            w = np.where(blend, alpha * T, F(0))
            for ch in range(3):
                if order == "base2":
                    Cc[ch] = ar.fma(w, np.full(P, col32[s, ch]), Cc[ch])
                else:
                    Cc[ch] = Cc[ch] + w * col32[s, ch]
            T = np.where(blend, Tn, T)
            nc = np.where(blend, j + 1, nc)
            done |= stop
            blended[j] = blend
            vs[j] = v
            als[j] = alpha
        for ch in range(3):
            image[ch, ys, xs] = ar.fma(T, np.full(P, bg[ch]), Cc[ch])
        Tout[ys, xs] = T
        ncout[ys, xs] = nc
        # backward: T recovered from T_final by faithful reciprocals, colour behind as GB
        g = [dldc[ch, ys, xs].astype(F) for ch in range(3)]
        gbg = ar.fma(g[0], np.full(P, bg[0]), ar.fma(g[1], np.full(P, bg[1]), g[2] * bg[2]))
        Tb = T.copy()
        Tfin = T.copy()
        GB = np.zeros(P, F)
        pid = (ys * W + xs).astype(np.int64)
        for j in range(n - 1, -1, -1):
            act = blended[j]
            if not act.any():
                continue
            s = lst[j]
            alpha = als[j]
            v = vs[j]
            inv = ar.rcp(F(1) - alpha)
            Tj = Tb * inv
            sgc = ar.fma(g[0], np.full(P, col32[s, 0]), ar.fma(g[1], np.full(P, col32[s, 1]), g[2] * col32[s, 2]))
            ge = sgc - GB
            dLda = Tj * ge
            if np.any(bg != 0):
                dLda = ar.fma(-Tfin * inv, gbg, dLda)
            wgt = alpha * Tj
            unclamped = v <= amax
            gv = np.where(unclamped, v * dLda, F(0))
            dx = pxc - m32[s, 0]
            dy = pyc - m32[s, 1]
            gx, gy = gv * dx, gv * dy
            vals9 = np.stack([gx, gy, gx * dx, gx * dy, gy * dy, gv, wgt * g[0], wgt * g[1], wgt * g[2]], 1)
            contrib.append((np.full(int(act.sum()), s), pid[act], vals9[act]))
            GB = np.where(act, ar.fma(alpha, ge, GB), GB)
            Tb = np.where(act, Tj, Tb)
    # per slot: sequential float32 sums in a random order of the contributions
    sl = np.concatenate([c[0] for c in contrib]) if contrib else np.zeros(0, np.int64)
    vv = np.concatenate([c[2] for c in contrib]) if contrib else np.zeros((0, 9), F)
    perm = ar.rng.permutation(sl.size)
    sl, vv = sl[perm], vv[perm]
    order_s = np.argsort(sl, kind="stable")
    sl, vv = sl[order_s], vv[order_s]
    sums = np.zeros((S, 9), F)
    counts = np.bincount(sl, minlength=S)
    starts = np.concatenate([[0], np.cumsum(counts)])
    kmax = int(counts.max()) if counts.size else 0
    for k in range(kmax):
        has = counts > k
        idx = starts[:-1][has] + k
        sums[has] = sums[has] + vv[idx]
    # the entry-constant factors, as a float32 rasterizer applies them to the summed parts
    ca = F(-0.5) * LOG2E
    a, b, c = ca * c32[:, 0], -LOG2E * c32[:, 1], ca * c32[:, 2]
    grad = np.zeros((S, 9), F)
    grad[:, 0] = -LN2 * ar.fma(F(2) * a, sums[:, 0], b * sums[:, 1])
    grad[:, 1] = -LN2 * ar.fma(b, sums[:, 0], F(2) * c * sums[:, 1])
    grad[:, 2] = sums[:, 2] * F(-0.5)
    grad[:, 3] = -sums[:, 3]
    grad[:, 4] = sums[:, 4] * F(-0.5)
    grad[:, 5] = np.where(sums[:, 5] != 0, sums[:, 5] / o32, F(0))
    grad[:, 6:9] = sums[:, 6:9]
    return image, Tout, ncout, grad, counts


def check_forward(f, img32, T32, nc32):
    """Unflagged pixels: same n_contrib, colour within err_C, T within err_T T.  Flagged pixels:
    equal to the base or to one of the oracle's alternatives within the same bounds."""
    C, T, nc = f["image"], f["T_final"], f["n_contrib"]
    eC, eT = f["err_C"], f["err_T"]
    okC = (np.abs(img32.astype(np.float64) - C) <= eC).all(0)
    okT = np.abs(T32.astype(np.float64) - T) <= eT * T
    ok = okC & okT & (nc32 == nc)
    assert not f["unresolved"].any()
    plain = ~f["flag"]
    assert ok[plain].all(), f"{int((~ok & plain).sum())} unflagged pixels outside the bounds"
    W = C.shape[2]
    alt = f["alt"]
    via_alt = 0
    for y, x in np.argwhere(f["flag"] & ~ok):
        k = np.nonzero(alt["pix"] == y * W + x)[0]
        good = [(np.abs(img32[:, y, x].astype(np.float64) - alt["C"][i]) <= eC[:, y, x]).all()
                and abs(float(T32[y, x]) - alt["T"][i]) <= eT[y, x] * alt["T"][i] and nc32[y, x] == alt["nc"][i]
                for i in k]
        assert any(good), f"flagged pixel ({x}, {y}) matches neither the base nor an alternative"
        via_alt += 1
    ratio = np.abs(img32.astype(np.float64) - C) / np.maximum(eC, 1e-300)
    return int(f["flag"].sum()), via_alt, float(ratio[:, plain].max())


def check_backward(b, grad32, counts):
    """Float32 gradients within err + (m + 6) u mag + widen, m = contributions summed."""
    tol = b["err"] + (counts[:, None] + 6) * U * b["mag"] + b["widen"]
    g64 = np.concatenate([b["d_mean2d"], b["d_conic"], b["d_opacity"][:, None], b["d_color"]], 1)
    err = np.abs(grad32.astype(np.float64) - g64)
    ok = err <= tol
    assert ok.all(), f"{int((~ok).sum())} gradient components outside the bound; worst {np.argwhere(~ok)[:3]}"
    nz = b["mag"] > 0
    return float((err[nz] / tol[nz]).max()) if nz.any() else 0.0


CASES = ["workload-4096", "random", "opaque-stack", "opaque-stack-bg"]


@pytest.mark.parametrize("order", ["definition", "base2"])
@pytest.mark.parametrize("case", CASES)
def test_compositing_error_bounds_cover_float32(oracle_mod, case, order):
    rng = np.random.default_rng(7)
    if case == "workload-4096":
        sc = scenes.make_scene(1)
        W, H, ranges, vals, recs, st = scene_records(oracle_mod, sc)
    elif case == "random":
        sc = scenes.random_scene(3000, 96, 80, seed=3, log_scale_mean=-2.6, opacity_std=1.5)
        W, H, ranges, vals, recs, st = scene_records(oracle_mod, sc)
    else:
        W, H, ranges, vals, recs = opaque_stack_records(rng)
        st = scenes.make_scene(1).settings(bg=(0.3, 0.6, 0.9) if case.endswith("bg") else (0.0, 0.0, 0.0))
    dldc = (0.8 * rng.choice([-1.0, 1.0], (3, H, W)) + 0.2 * rng.standard_normal((3, H, W))).astype(F)
    f = oracle_mod.raster_forward(W, H, ranges, vals, recs, st)
    b = oracle_mod.raster_backward(W, H, ranges, vals, recs, st, dldc.astype(np.float64))
    assert not b["slot_flag"].any()
    worst_px, worst_g = 0.0, 0.0
    n_flag = n_alt = 0
    for seed in range(3):
        img32, T32, nc32, g32, counts = emulate(oracle_mod, W, H, ranges, vals, recs, st, order, seed, dldc)
        nf, na, wp = check_forward(f, img32, T32, nc32)
        n_flag, n_alt = nf, n_alt + na
        worst_px = max(worst_px, wp)
        worst_g = max(worst_g, check_backward(b, g32, counts))
    blended = f["n_blended"]
    print(f"[error model] {case} {order}: {blended} blends, {n_flag} flagged pixels "
          f"({n_alt} float32 evaluations matched an alternative); worst colour error / err_C {worst_px:.3f}; "
          f"worst gradient error / bound {worst_g:.3f}")
    if case.startswith("opaque"):
        assert f["n_clamped"] > 0 and (f["T_final"] < 1e-3).mean() > 0.5  # the stress the case is for
    # not vacuous: colour bounds within a factor 64 of the worst error seen, and small in
    # relative terms where the colour is not tiny
    assert worst_px >= 1.0 / 64
    C = f["image"]
    big = C > 1e-2
    assert np.median(f["err_C"][big] / C[big]) <= 0.5e-5


# ------------------------------------------------------------------------------------------
# decisions on their thresholds: the alternatives
# ------------------------------------------------------------------------------------------
def on_threshold_records(rng, kind):
    """Records whose decision at pixel (8, 8) sits within ~1e-9 (relative) of its threshold in
    fp64, so that float32 evaluation takes it either way:
      amin: one isotropic splat, o exp(-q/2) = alpha_min at that pixel (then blended or skipped);
      tmin: three near-opaque splats centred on the pixel whose T after the third is t_min
            (then the third is blended or the pixel stops);
    plus a splat behind, so that the decision changes what follows."""
    amin, tmin = 1.0 / 255.0, 1e-4
    best = None
    for _ in range(20000):
        if kind == "amin":
            o = F(rng.uniform(0.3, 0.9))
            d = F(rng.uniform(2.0, 3.0))
            A = F(2.0 * np.log(float(o) / amin) / float(d) ** 2)
            # as the oracle evaluates it, from the float32 records widened
            v = float(o) * np.exp(-0.5 * float(A) * float(d) ** 2)
            gap = abs(v / amin - 1.0)
            rec = dict(mean2d=[[8.5 - float(d), 8.5], [8.5, 8.5]], conic=[[float(A), 0.0, float(A)], [0.05, 0.0, 0.05]],
                       opacity=[float(o), 0.7], color=[[0.9, 0.2, 0.4], [0.1, 0.8, 0.3]])
        else:
            # centres slightly off the pixel, so that every alpha carries an exponential
            cen = [[8.5 - 0.3, 8.5 + 0.2], [8.5 + 0.25, 8.5], [8.5, 8.5 - 0.35]]
            con = [F(0.05), F(0.0), F(0.05)]
            q = [float(con[0]) * ((8.5 - float(F(c[0]))) ** 2 + (8.5 - float(F(c[1]))) ** 2) for c in cen]
            o1, o2 = F(rng.uniform(0.95, 0.97)), F(rng.uniform(0.95, 0.97))
            a1 = float(o1) * np.exp(-0.5 * q[0])
            a2 = float(o2) * np.exp(-0.5 * q[1])
            tmin32 = float(F(tmin))
            o3 = F((1.0 - tmin32 / ((1.0 - a1) * (1.0 - a2))) / np.exp(-0.5 * q[2]))
            a3 = float(o3) * np.exp(-0.5 * q[2])
            T3 = (1.0 - a1) * (1.0 - a2) * (1.0 - a3)
            gap = abs(T3 / tmin32 - 1.0)
            rec = dict(mean2d=cen + [[8.5, 8.5]], conic=[[float(c) for c in con]] * 4,
                       opacity=[float(o1), float(o2), float(o3), 0.6],
                       color=[[0.9, 0.2, 0.4], [0.1, 0.8, 0.3], [0.5, 0.5, 0.1], [0.3, 0.3, 0.9]])
        if best is None or gap < best[0]:
            best = (gap, rec)
        if gap < 2e-9:
            break
    gap, rec = best
    assert gap < 1e-8
    recs = {k: np.asarray(v, np.float64) for k, v in rec.items()}
    recs = f32_records(recs)
    n = recs["opacity"].size
    vals = np.arange(n, dtype=np.int32)
    ranges = np.array([[0, n]], np.int32)
    return 16, 16, ranges, vals, recs


@pytest.mark.parametrize("order", ["definition", "base2"])
@pytest.mark.parametrize("kind", ["amin", "tmin"])
def test_alternatives_cover_flipped_decisions(oracle_mod, kind, order):
    """The oracle flags the on-threshold decision, its alternative takes it the other way, and
    float32 evaluations (over many rounding choices) land on the base or on the alternative,
    both of which occur; the backward's widening covers the gradients either way."""
    rng = np.random.default_rng(5 if kind == "amin" else 6)
    st = scenes.make_scene(1).settings()
    seen_base = seen_alt = 0
    for case in range(8):
        # each construction has its own fixed rounding biases: several, so that float32 lands
        # on both sides of the threshold
        W, H, ranges, vals, recs = on_threshold_records(rng, kind)
        f = oracle_mod.raster_forward(W, H, ranges, vals, recs, st)
        assert f["flag"][8, 8] and not f["unresolved"].any()
        k = np.nonzero(f["alt"]["pix"] == 8 * W + 8)[0]
        assert k.size >= 1
        base_nc = int(f["n_contrib"][8, 8])
        assert any(int(f["alt"]["nc"][i]) != base_nc or abs(f["alt"]["T"][i] - f["T_final"][8, 8]) > 1e-6 for i in k)
        dldc = np.ones((3, H, W))
        b = oracle_mod.raster_backward(W, H, ranges, vals, recs, st, dldc)
        assert b["stats"]["flagged_pixels"] >= 1 and b["widen"].max() > 0
        for seed in range(10):
            img32, T32, nc32, g32, counts = emulate(oracle_mod, W, H, ranges, vals, recs, st, order, seed,
                                                    dldc.astype(F))
            _, via_alt, _ = check_forward(f, img32, T32, nc32)
            check_backward(b, g32, counts)
            seen_alt += via_alt
            seen_base += via_alt == 0
    print(f"[error model] on-threshold {kind} {order}: float32 took the base decisions {seen_base} times, "
          f"an alternative {seen_alt} times")
    assert seen_alt > 0 and seen_base > 0
