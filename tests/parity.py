"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Comparison contract (stage-isolated, so that every integer result is compared bit for bit):
  * projection: visible sets equal up to Gaussians whose decision the oracle flags as within
    float32 reach; records within the float tolerances below;
  * binning and cap: the oracle's NumPy binning run on the GPU's own projected records must
    reproduce tile keys, order, ranges and capped lists exactly;
  * forward: the oracle composites the GPU's records over the GPU's lists in double
    precision; image and T_final within 1e-5 relative + 1e-7 absolute, n_contrib exact, on
    pixels whose decisions are not within float32 reach; for the image, plus the oracle's
    first-order float32 error bound of the pixel (large only behind near-opaque splats, where
    1 / (1 - alpha) amplifies the rounding of alpha), with the count of components that pass
    only through it reported;
  * backward: gradients within 1e-3 relative + 1e-6 absolute on slots that no flagged pixel
    blends (dL/dC scaled to O(1): L1 summed, scale 1), plus 1e-5 times the summed magnitude of
    the component's contributions, which bounds float32 error when the contributions cancel;
    the report counts the comparisons that pass only through that term.
"""
import numpy as np

EPS32 = 2.0 ** -24
IMG_RTOL, IMG_ATOL = 1e-5, 1e-7
IMG_COND_FACTOR = 1.0  # times the oracle's float32 error bound of the pixel colour
GRAD_RTOL, GRAD_ATOL = 1e-3, 1e-6
GRAD_MAG_TOL = 1e-5  # times the summed |contributions| of a gradient component


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
    sel = pixel_mask(cam, region) & ~f["flag"]
    go, oo = img_g[:, sel].astype(np.float64), f["image"][:, sel]
    strict = close(go, oo, IMG_RTOL, IMG_ATOL)
    # conditioning: behind a near-opaque splat the float32 rounding of alpha is amplified by
    # 1 / (1 - alpha) in T; the oracle's first-order float32 error bound err_C covers it
    cond = IMG_COND_FACTOR * f["err_C"][sel][None, :]
    ok_img = np.abs(go - oo) <= IMG_RTOL * np.abs(oo) + IMG_ATOL + cond
    nflag = int((pixel_mask(cam, region) & f["flag"]).sum())
    bad = report("image", ok_img, f"({nflag} flagged pixels skipped; {int((ok_img & ~strict).sum())} within "
                                  f"tolerance only through the conditioning term)")
    if T_g is not None:
        To = f["T_final"][sel]
        ok_T = np.abs(T_g[sel].astype(np.float64) - To) <= IMG_RTOL * To + IMG_ATOL + \
            IMG_COND_FACTOR * f["err_T"][sel] * To
        ok_nc = nc_g[sel] == f["n_contrib"][sel]
        bad += report("T_final", ok_T) + report("n_contrib", ok_nc)
    if bad:
        err = np.abs(go - oo)
        worst = np.unravel_index(np.argmax(err / (IMG_RTOL * np.abs(oo) + IMG_ATOL + cond)), err.shape)
        print(f"[parity] worst image component: gpu {go[worst]:.9g} oracle {oo[worst]:.9g} "
              f"err {err[worst]:.3g} err_C {f['err_C'][sel][worst[1]]:.3g}", flush=True)
    assert bad == 0
    return f


def compare_backward(oracle, cam, settings, rec, ranges, vals, dldc, grads_g, fwd_o, region=None, extra_skip=None,
                     slots_rect=None):
    r = region_ranges(ranges, cam.tiles_x, region)
    skip = fwd_o["flag"].copy()
    if extra_skip is not None:
        skip |= extra_skip
    b = oracle.raster_backward(cam.width, cam.height, r, vals, rec, settings, dldc, pixel_skip=skip)
    S = rec["opacity"].shape[0]
    use = ~b["slot_flag"]
    if region is not None:
        # only slots whose whole tile rectangle lies inside the region have complete gradients
        tx0, ty0, tx1, ty1 = region
        rc = slots_rect
        use &= (rc[:, 0] >= tx0) & (rc[:, 2] <= tx1) & (rc[:, 1] >= ty0) & (rc[:, 3] <= ty1)
    total_bad = 0
    mag_cols = {"d_mean2d": [0, 1], "d_conic": [2, 3, 4], "d_opacity": [5], "d_color": [6, 7, 8]}
    for key, k in [("d_mean2d", 2), ("d_conic", 3), ("d_opacity", 1), ("d_color", 3)]:
        go = b[key].reshape(S, k)[use]
        gg = grads_g[key].reshape(S, k)[use].astype(np.float64)
        mag = b["mag"][:, mag_cols[key]][use]
        strict = close(gg, go, GRAD_RTOL, GRAD_ATOL)
        # cancellation: the float32 sum of contributions whose magnitudes add up to `mag`
        # carries an error proportional to mag, not to the (possibly much smaller) result
        ok = np.abs(gg - go) <= GRAD_RTOL * np.abs(go) + GRAD_ATOL + GRAD_MAG_TOL * mag
        bad = report(key, ok, f"({int((~use).sum())} slots skipped; {int((ok & ~strict).sum())} within "
                              f"tolerance only through the cancellation term)")
        if bad:
            i = np.argwhere(~ok)[:5]
            for (s, c) in i:
                print(f"    slot {s} comp {c}: gpu {gg[s, c]:.9g} oracle {go[s, c]:.9g}", flush=True)
        total_bad += bad
    assert total_bad == 0
    return b


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
    params = oracle.scene_params_f64(scene)
    n_all = scene.n
    idx = np.arange(n_all) if sample is None else np.asarray(sample)
    if sample is not None:
        params = {k: np.ascontiguousarray(v[..., idx]) for k, v in params.items()}
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
