"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Comparison contract (stage-isolated, so that every integer result is compared bit for bit):
  * projection: visible sets equal up to Gaussians whose decision the oracle flags as within
    float32 reach; records within the float tolerances below;
  * binning and cap: the oracle's NumPy binning run on the GPU's own projected records must
    reproduce tile keys, order, ranges and capped lists exactly;
  * forward: the oracle composites the GPU's records over the GPU's lists in double precision;
    image and T_final within 1e-5 relative + 1e-7 absolute, plus the oracle's float32 error
    bound of the pixel (err_C per channel, err_T T; pinned against float32 evaluations of the
    compositing); n_contrib exact.  A pixel with decisions within float32 reach of their
    thresholds (alpha_min, t_min) must match the base or one of the oracle's alternatives (the
    same pixel with any combination of those decisions taken the other way).  Asserted: every
    compared pixel matches; flagged pixels are fewer than 1e-4 of the pixels (at least 4 are
    allowed on small images); no more than 1e-5 of the pixels are left uncompared (more than
    three flagged decisions); at most 1e-4 of the image components (at least one) pass only
    through the error bound;
  * backward: gradients within 1e-3 relative + 1e-6 absolute (dL/dC of O(1): L1 summed, scale
    1), plus twice the oracle's float32 bound (the summed running error bounds of the
    contributions and the rounding of their sum, depth times u times their summed magnitude,
    with the depth of the rasterizer's reduction: a 16-lane tree, up to 16 blocks of a tile in
    sequence, the slot's instance records in sequence, the final factors), plus the oracle's
    widening where flagged decisions (and unsure L1 signs) can change a contribution.
    Asserted: every compared component matches; at most 1e-4 of the components of each kind
    (at least one) pass only through the bound; at most 1e-3 of the slots are left uncompared.
"""
from types import SimpleNamespace

import numpy as np

EPS32 = 2.0 ** -24
IMG_RTOL, IMG_ATOL = 1e-5, 1e-7
GRAD_RTOL, GRAD_ATOL = 1e-3, 1e-6
GRAD_BOUND_FACTOR = 2.0  # times the oracle's float32 error bound of a gradient component
FLAG_FRACTION = 1e-4     # flagged pixels must be fewer than this fraction of the pixels
ONLY_BOUND_FRACTION = 1e-4  # comparisons passing only through the float32 bound
# depth of the rasterizer's float32 reduction of a slot's contributions, beyond its records:
# 4 levels of a 16-lane tree, up to 16 blocks of a tile summed in sequence, 4 roundings of the
# final factors; the records of the slot's instances are summed in sequence on top
REDUCTION_DEPTH = 24


def close(a, b, rtol, atol):
    return np.abs(a - b) <= rtol * np.abs(b) + atol


def report(name, ok, extra=""):
    bad = int((~ok).sum())
    print(f"[parity] {name}: {ok.size - bad}/{ok.size} within tolerance {extra}", flush=True)
    return bad


def compare_projection(oracle, scene, cam, settings, gpu: dict):
    """A1 end-to-end from the raw parameters."""
    proj = oracle.project(scene, cam, settings)
    vis_o = np.nonzero(proj["visible"])[0]
    vis_g = gpu["vis_ids"]
    assert np.all(np.diff(vis_g) > 0), "slots must follow ascending Gaussian index"
    diff = np.setxor1d(vis_o, vis_g)
    unexplained = diff[proj["flag"][diff] == 0]
    assert unexplained.size == 0, f"visibility differs for unflagged Gaussians {unexplained[:10]}"
    common, io, ig = np.intersect1d(vis_o, vis_g, return_indices=True)
    keep = proj["flag"][common] == 0
    o_idx = common[keep]
    g_sel = ig[keep]
    # float records
    m_o = proj["mean2d"][o_idx]
    m_g = gpu["mean2d"][g_sel].astype(np.float64)
    # the camera transform R mu + t cancels terms of size |R||mu| + |t|; float32 leaves an
    # absolute error of a few ulp of that size in (tx, tz), which f / tz turns into pixels
    R = cam.R.astype(np.float64)
    t = cam.t.astype(np.float64)
    mu = scene.means[:, o_idx].astype(np.float64)
    size = np.abs(R) @ np.abs(mu) + np.abs(t)[:, None]          # (3, n)
    tz = proj["depth"][o_idx]
    tc_x = (R[0] @ mu + t[0], R[1] @ mu + t[1])
    cond = np.stack([cam.fx / tz * (size[0] + np.abs(tc_x[0]) / tz * size[2]),
                     cam.fy / tz * (size[1] + np.abs(tc_x[1]) / tz * size[2])], 1)
    tol_m = 2e-4 + 1e-6 * np.abs(m_o) + 8 * EPS32 * cond
    bad_m = np.abs(m_g - m_o) > tol_m
    assert not bad_m.any(), f"mean2d: {int(bad_m.any(1).sum())} off, worst {float((np.abs(m_g - m_o) / tol_m).max())}"
    cov = proj["cov2d"][o_idx]
    kappa = (np.abs(cov[:, 0] * cov[:, 2]) + cov[:, 1] ** 2) / (cov[:, 0] * cov[:, 2] - cov[:, 1] ** 2)
    conic_o = proj["conic"][o_idx]
    conic_g = gpu["conic_opacity"][g_sel, :3].astype(np.float64)
    scale = np.maximum(np.abs(conic_o[:, 0]), np.abs(conic_o[:, 2]))[:, None]
    tol = (1e-5 + 64 * EPS32 * kappa)[:, None] * scale
    bad_conic = ~(np.abs(conic_g - conic_o) <= tol)
    assert not bad_conic.any(), f"conic: {int(bad_conic.any(1).sum())} Gaussians off"
    assert close(gpu["conic_opacity"][g_sel, 3].astype(np.float64), proj["opacity"][o_idx], 1e-6, 1e-7).all(), "opacity"
    assert close(gpu["color"][g_sel].astype(np.float64), proj["color"][o_idx], 1e-5, 1e-5).all(), "color"
    assert close(gpu["depth"][g_sel].astype(np.float64), proj["depth"][o_idx], 1e-6, 0).all(), "depth"
    assert np.array_equal(gpu["rect"][g_sel], proj["rect"][o_idx]), "tile rect"
    assert np.array_equal(gpu["n_tiles"][g_sel], proj["n_tiles"][o_idx]), "n_tiles"
    print(f"[parity] projection: {vis_g.size} visible, {diff.size} flagged differences, "
          f"{int((proj['flag'][common] != 0).sum())} flagged in common", flush=True)
    return proj


def gpu_records(gpu: dict) -> dict:
    """The GPU's float32 records, widened exactly to float64 for the oracle."""
    co = gpu["conic_opacity"].astype(np.float64)
    return dict(mean2d=gpu["mean2d"].astype(np.float64), conic=co[:, :3].copy(), opacity=co[:, 3].copy(),
                color=gpu["color"].astype(np.float64))


def compare_binning(oracle, cam, gpu: dict, bins_g: dict):
    """A2-A5 stage-isolated: oracle binning of the GPU's own rect / n_tiles / depth."""
    dbits = gpu["depth"].view(np.uint32)
    b = oracle.bin_tiles(gpu["rect"], gpu["n_tiles"], dbits, cam.tiles_x, cam.tiles_y)
    assert b["num_instances"] == gpu["inst_count"] == bins_g["vals"].size, "instance count"
    assert np.array_equal(bins_g["vals"], b["vals"]), "sorted slots"
    assert np.array_equal(bins_g["tile_keys"].astype(np.int64), (b["keys"] >> np.uint64(32)).astype(np.int64)), "keys"
    assert np.array_equal(bins_g["ranges"], b["ranges"]), "ranges"
    return b


def compare_cap(oracle, gpu: dict, b: dict, capped_g: dict, K: int):
    score = oracle.cap_score(gpu["conic_opacity"][:, :3], gpu["conic_opacity"][:, 3])
    c = oracle.cap_tiles(b["ranges"], b["vals"], score, gpu["depth"].view(np.uint32), K)
    if not (np.array_equal(capped_g["vals"], c["vals"]) and np.array_equal(capped_g["ranges"], c["ranges"])):
        dbits = gpu["depth"].view(np.uint32)
        for t in range(b["ranges"].shape[0]):
            go = capped_g["vals"][capped_g["ranges"][t, 0]:capped_g["ranges"][t, 1]]
            oo = c["vals"][c["ranges"][t, 0]:c["ranges"][t, 1]]
            if not np.array_equal(go, oo):
                full = b["vals"][b["ranges"][t, 0]:b["ranges"][t, 1]]
                only_g = np.setdiff1d(go, oo)
                only_o = np.setdiff1d(oo, go)
                print(f"[cap] tile {t}: n={full.size} K={K} gpu kept {go.size} oracle kept {oo.size}; "
                      f"gpu-only {only_g[:5]} scores {score[only_g[:5]].view(np.uint32)} depth {dbits[only_g[:5]]}; "
                      f"oracle-only {only_o[:5]} scores {score[only_o[:5]].view(np.uint32)} depth {dbits[only_o[:5]]}",
                      flush=True)
                sc = score[full].view(np.uint32)
                kth = np.sort(sc)[::-1][K - 1]
                print(f"[cap]   K-th best score bits {kth}; entries with those bits {int((sc == kth).sum())}", flush=True)
                break
    assert np.array_equal(capped_g["vals"], c["vals"]), "capped slots"
    assert np.array_equal(capped_g["ranges"], c["ranges"]), "capped ranges"
    return c


def region_ranges(ranges: np.ndarray, tiles_x: int, region):
    """Keep only the tiles of region = (tx0, ty0, tx1, ty1) inclusive (others empty)."""
    if region is None:
        return ranges
    r = np.zeros_like(ranges)
    tx0, ty0, tx1, ty1 = region
    for ty in range(ty0, ty1 + 1):
        for tx in range(tx0, tx1 + 1):
            r[ty * tiles_x + tx] = ranges[ty * tiles_x + tx]
    return r


def pixel_mask(cam, region):
    m = np.zeros((cam.height, cam.width), bool)
    if region is None:
        m[:] = True
        return m
    tx0, ty0, tx1, ty1 = region
    m[ty0 * 16:min(cam.height, (ty1 + 1) * 16), tx0 * 16:min(cam.width, (tx1 + 1) * 16)] = True
    return m


def compare_forward(oracle, cam, settings, rec, ranges, vals, img_g, T_g, nc_g, region=None):
    """T_g / nc_g may be None (the fused kernel returns only the image)."""
    r = region_ranges(ranges, cam.tiles_x, region)
    f = oracle.raster_forward(cam.width, cam.height, r, vals, rec, settings)
    reg = pixel_mask(cam, region)
    npx = int(reg.sum())
    sel = reg & ~f["unresolved"]
    go, oo, eC = img_g.astype(np.float64), f["image"], f["err_C"]
    tolC = IMG_RTOL * np.abs(oo) + IMG_ATOL
    strict = np.abs(go - oo) <= tolC
    okC = np.abs(go - oo) <= tolC + eC
    ok = okC.all(0)
    if T_g is not None:
        To, eT = f["T_final"], f["err_T"]
        ok &= np.abs(T_g.astype(np.float64) - To) <= IMG_RTOL * To + IMG_ATOL + eT * To
        ok &= nc_g == f["n_contrib"]
    # flagged pixels that differ from the base: the alternatives
    alt = f["alt"]
    via_alt = 0
    W = cam.width
    for y, x in np.argwhere(sel & f["flag"] & ~ok):
        for i in np.nonzero(alt["pix"] == y * W + x)[0]:
            a_ok = (np.abs(go[:, y, x] - alt["C"][i]) <= IMG_RTOL * np.abs(alt["C"][i]) + IMG_ATOL + eC[:, y, x]).all()
            if T_g is not None:
                Ta = alt["T"][i]
                a_ok &= abs(float(T_g[y, x]) - Ta) <= IMG_RTOL * Ta + IMG_ATOL + f["err_T"][y, x] * Ta
                a_ok &= int(nc_g[y, x]) == int(alt["nc"][i])
            if a_ok:
                ok[y, x] = True
                via_alt += 1
                break
    bad = int((sel & ~ok).sum())
    n_flag = int((reg & f["flag"]).sum())
    n_unres = int((reg & f["unresolved"]).sum())
    plain = sel & ~f["flag"]
    n_cond = int((okC & ~strict)[:, plain].sum())
    n_comp = 3 * int(plain.sum())
    print(f"[parity] image{'/T_final/n_contrib' if T_g is not None else ''}: {int(sel.sum()) - bad}/{int(sel.sum())} "
          f"pixels match; {n_flag} flagged pixels ({n_flag / max(npx, 1):.1e}; {via_alt} matched an alternative), "
          f"{n_unres} uncompared; {n_cond} of {n_comp} components within tolerance only through the float32 bound",
          flush=True)
    if bad:
        err = np.abs(go - oo)
        worst = np.unravel_index(np.argmax(np.where(sel[None], err / (tolC + eC), 0)), err.shape)
        print(f"[parity] worst image component {worst}: gpu {go[worst]:.9g} oracle {oo[worst]:.9g} "
              f"err {err[worst]:.3g} err_C {eC[worst]:.3g}", flush=True)
        if T_g is not None:
            for y, x in np.argwhere(sel & ~ok)[:5]:
                print(f"    pixel ({x}, {y}): T gpu {T_g[y, x]:.9g} oracle {f['T_final'][y, x]:.9g}; n_contrib gpu "
                      f"{nc_g[y, x]} oracle {f['n_contrib'][y, x]}", flush=True)
    assert bad == 0
    assert n_flag <= max(FLAG_FRACTION * npx, 4), ("flagged pixels", n_flag, npx)
    assert n_unres <= 1e-5 * npx, ("uncompared pixels", n_unres)
    assert n_cond <= max(1, ONLY_BOUND_FRACTION * n_comp), ("image components only through the bound", n_cond)
    return f


def rect_tiles(rect):
    rc = np.asarray(rect).astype(np.int64)
    return (rc[:, 2] - rc[:, 0] + 1) * (rc[:, 3] - rc[:, 1] + 1)


def compare_backward(oracle, cam, settings, rec, ranges, vals, dldc, grads_g, dg=None, region=None, slots_rect=None):
    """dg: the oracle's uncertainty of dL/dC (unsure L1 signs), widening the comparison."""
    r = region_ranges(ranges, cam.tiles_x, region)
    b = oracle.raster_backward(cam.width, cam.height, r, vals, rec, settings, dldc, dg=dg)
    S = rec["opacity"].shape[0]
    use = ~b["slot_flag"]
    n_unres = int(b["slot_flag"].sum())
    if region is not None:
        # only slots whose whole tile rectangle lies inside the region have complete gradients
        tx0, ty0, tx1, ty1 = region
        rc = slots_rect
        use &= (rc[:, 0] >= tx0) & (rc[:, 2] <= tx1) & (rc[:, 1] >= ty0) & (rc[:, 3] <= ty1)
    depth = REDUCTION_DEPTH + rect_tiles(slots_rect).astype(np.float64)
    bound = GRAD_BOUND_FACTOR * (b["err"] + depth[:, None] * EPS32 * b["mag"])
    widen = b["widen"]
    total_bad = 0
    cols = {"d_mean2d": [0, 1], "d_conic": [2, 3, 4], "d_opacity": [5], "d_color": [6, 7, 8]}
    n_widen_total = 0
    for key, k in [("d_mean2d", 2), ("d_conic", 3), ("d_opacity", 1), ("d_color", 3)]:
        go = b[key].reshape(S, k)[use]
        gg = grads_g[key].reshape(S, k)[use].astype(np.float64)
        bd = bound[:, cols[key]][use]
        wd = widen[:, cols[key]][use]
        err = np.abs(gg - go)
        base = GRAD_RTOL * np.abs(go) + GRAD_ATOL
        strict = err <= base
        ok_bound = err <= base + bd
        ok = err <= base + bd + wd
        n_bound = int((ok_bound & ~strict).sum())
        n_widen = int((ok & ~ok_bound).sum())
        n_widen_total += n_widen
        rel = err / (np.abs(go) + 1e-30)
        q = np.quantile(rel, [0.5, 0.99]) if rel.size else [0, 0]
        bad = report(key, ok, f"({n_bound} within tolerance only through the float32 bound, {n_widen} only through "
                              f"the flagged decisions' widening; relative error median {q[0]:.2g} p99 {q[1]:.2g})")
        if bad:
            for (s_, c_) in np.argwhere(~ok)[:5]:
                print(f"    slot {s_} comp {c_}: gpu {gg[s_, c_]:.9g} oracle {go[s_, c_]:.9g} bound {bd[s_, c_]:.3g} "
                      f"widen {wd[s_, c_]:.3g}", flush=True)
        total_bad += bad
        assert n_bound <= max(1, ONLY_BOUND_FRACTION * ok.size), (key, "only through the bound", n_bound)
    print(f"[parity] backward: {int(use.sum())} of {S} slots compared, {n_unres} left out (unresolved pixels); "
          f"{b['stats']['flagged_pixels']} pixels with flagged decisions", flush=True)
    assert total_bad == 0
    assert n_unres <= 1e-3 * S, ("slots left out", n_unres, S)
    return b


def compare_loss_grad_l1(oracle, img_o, target, scale, err_C, dl_g):
    """The separate path's L1 gradient kernel against the oracle's: equal wherever the sign is
    not within float32 reach; elsewhere one of -scale, 0, scale.  Returns (g, dg) for the
    backward comparison."""
    g, dg = oracle.loss_grad_l1(img_o, target, scale, err_C)
    sure = dg == 0
    dl = np.asarray(dl_g, np.float64)
    assert np.array_equal(dl[sure], g[sure]), "L1 gradient differs where its sign is certain"
    assert np.isin(dl[~sure], [-scale, 0.0, scale]).all()
    print(f"[parity] L1 gradient: {int(sure.sum())}/{sure.size} components equal; {int((~sure).sum())} with a sign "
          f"within float32 reach", flush=True)
    return g, dg


def slot_to_gaussian(n, vis_ids, arr, k):
    """Scatter a per-slot array (slots, k) into a per-Gaussian float64 array (n, k) (zeros elsewhere)."""
    out = np.zeros((n, k))
    out[vis_ids] = np.asarray(arr, np.float64).reshape(-1, k)[: vis_ids.size]
    return out


def compare_project_backward(oracle, scene, settings, views, grads2d_g, grads3d_g, sample=None):
    """Projection backward, stage-isolated: the oracle chains the GPU's own per-slot 2D gradients
    of every view (and the GPU's visible sets) to the parameters in double precision.

    views: list of (camera, vis_ids) per view; grads2d_g: per view the dict of grads_host();
    grads3d_g: dict of grads3d_host(); sample: optional Gaussian indices (the oracle then runs on
    that subset only, with the GPU's outputs gathered at them).
    Contract per component: within 1e-3 relative + 1e-6 absolute plus twice the oracle's
    first-order bound on the error of a float32 evaluation of the same chain (large only where
    the chain's terms cancel: scale and rotation gradients of Gaussians elongated along the
    view direction); and at most 1e-4 of the components of each kind may need that bound term.
    Colour and mean gradients of Gaussians whose colour sits within float32 reach of the clamp at
    zero in some view are skipped."""
    n_all = scene.n
    idx = np.arange(n_all) if sample is None else np.asarray(sample)
    if sample is None:
        params = oracle.scene_params_f64(scene)
    else:
        # widen only the sampled Gaussians (a 40M scene's parameters are 19 GB in float64)
        params = oracle.scene_params_f64(SimpleNamespace(
            means=scene.means[:, idx], log_scales=scene.log_scales[:, idx], quats=scene.quats[:, idx],
            opacity_logits=scene.opacity_logits[idx], sh=scene.sh[:, idx]))
    n = idx.size
    acc = None
    for (cam, vis_ids), g2 in zip(views, grads2d_g):
        def per_gauss(key, k):
            full = slot_to_gaussian(n_all, vis_ids, g2[key], k)
            return full[idx]
        vis_full = np.zeros(n_all, np.int8)
        vis_full[vis_ids] = 1
        acc = oracle.project_backward(params, cam, settings, vis_full[idx], per_gauss("d_mean2d", 2),
                                      per_gauss("d_conic", 3), per_gauss("d_opacity", 1)[:, 0],
                                      per_gauss("d_color", 3), acc=acc, error_bound=True)
    flag = acc["flag"]
    bad_total = 0
    for key in ("d_means", "d_log_scales", "d_quats", "d_opacity_logits", "d_sh"):
        go = acc[key]
        eb = acc["e" + key[1:]]
        gg = np.asarray(grads3d_g[key], np.float64)[..., idx]
        use = np.ones(n, bool) if key not in ("d_means", "d_sh") else (flag == 0)
        go_u, gg_u, eb_u = go[..., use], gg[..., use], eb[..., use]
        err = np.abs(gg_u - go_u)
        base = GRAD_RTOL * np.abs(go_u) + GRAD_ATOL
        strict = err <= base
        ok = err <= base + 2.0 * eb_u
        n_bound = int((ok & ~strict).sum())
        rel = err / (np.abs(go_u) + 1e-30)
        q = np.quantile(rel, [0.5, 0.99]) if rel.size else [0, 0]
        bad = report(key, ok, f"({int((~use).sum())} Gaussians skipped at the colour clamp; {n_bound} within "
                              f"tolerance only through the float32 error bound; relative error median "
                              f"{q[0]:.2g} p99 {q[1]:.2g})")
        if bad:
            for loc in np.argwhere(~ok)[:5]:
                loc = tuple(loc)
                print(f"    {key}{loc}: gpu {gg_u[loc]:.9g} oracle {go_u[loc]:.9g} bound {eb_u[loc]:.3g}", flush=True)
        bad_total += bad
        assert n_bound <= max(1, 1e-4 * ok.size), (key, n_bound)
    assert bad_total == 0
    return acc
