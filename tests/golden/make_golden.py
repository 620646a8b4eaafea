"""Write the stored expected values of tests/golden/*.json.

The values come from the CPU oracle (oracle/, test infrastructure) and nothing else: this script
builds a small hand-specified scene, runs the oracle's full iteration on it (projection,
binning, compositing, L1 loss gradient, backward, projection backward summed over the views)
and stores a selection of the results.  The pages print no worked example of these
computations, so the fixture is a regression record of the oracle (its tests pin the oracle to
closed forms, brute force and finite differences) and a fixed target for the GPU path.

Run from the repository root: python tests/golden/make_golden.py
"""
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from differentiable_raster_amd import scenes  # noqa: E402  (input generators only)

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURE = os.path.join(HERE, "tiny_two_views.json")
# pixels whose colour, transmittance and n_contrib are stored (x, y); the rest enter through the
# per-channel sums
SAMPLE_PIXELS = [(x, y) for y in range(1, 32, 5) for x in range(2, 48, 7)]


def golden_scene() -> scenes.Scene:
    """40 Gaussians, 48x32 pixels, two views, SH degree 1, L1 against a constant target.

    Every value is a closed formula of the index k (no random draws): a front cluster stacked at
    the image centre (long lists, transmittance recursion, a near-opaque Gaussian at the alpha
    clamp), a spread of small ones, one wide Gaussian over several tiles, and Gaussians that the
    near plane and the frustum cull."""
    n = 40
    f32 = np.float32
    k = np.arange(n, dtype=np.float64)
    means = np.stack([0.05 * np.sin(1.7 * k) + 0.35 * ((k % 7) - 3) / 3.0 * (k >= 12),
                      0.05 * np.cos(1.3 * k) + 0.25 * ((k % 5) - 2) / 2.0 * (k >= 12),
                      2.0 + 0.08 * k])
    log_scales = np.stack([-2.6 + 0.3 * np.sin(0.9 * k), -2.7 + 0.25 * np.cos(1.1 * k), -2.8 + 0.1 * np.sin(k)])
    quats = np.stack([1.0 + 0.0 * k, 0.3 * np.sin(0.7 * k), -0.2 * np.cos(0.5 * k), 0.1 * np.sin(1.9 * k)])
    quats /= np.linalg.norm(quats, axis=0)
    logits = 0.8 * np.sin(2.3 * k) - 0.2
    logits[3] = 6.0            # o = 0.9975 > alpha_max: the clamp
    log_scales[:, 20] = -1.2   # wide: several tiles
    means[:, 36] = (0.0, 0.0, 0.1)    # in front of the near plane: culled
    means[:, 37] = (0.0, 0.0, -3.0)   # behind the camera
    means[:, 38] = (30.0, 0.0, 3.0)   # far outside the frustum
    means[:, 39] = (0.0, -25.0, 4.0)
    sh = np.zeros((12, n))
    sh[0] = 0.2 + 0.6 * (0.5 + 0.5 * np.sin(0.8 * k))
    sh[1] = 0.2 + 0.6 * (0.5 + 0.5 * np.cos(1.4 * k))
    sh[2] = 0.2 + 0.6 * (0.5 + 0.5 * np.sin(2.1 * k + 1.0))
    for c in range(3, 12):
        sh[c] = 0.15 * np.sin(0.6 * k + c)
    cams = [scenes.identity_camera(48, 32),
            scenes.look_at_camera(48, 32, (0.4, -0.2, -0.3), (0.0, 0.0, 3.0), (0.0, 1.0, 0.0))]
    target = np.full((2, 3, 32, 48), 0.3, f32)
    return scenes.Scene("golden-40-48x32-2v", means.astype(f32), log_scales.astype(f32), quats.astype(f32),
                        logits.astype(f32), sh.astype(f32), 1, cams, "l1", target, None)


def oracle_results(oracle, sc):
    """The oracle's iteration and projection backward on the golden scene."""
    st = sc.settings()
    it = oracle.iteration(sc, st, loss_scale=1.0)
    params = oracle.scene_params_f64(sc)
    acc = None
    n = sc.n
    views = []
    for r in it:
        rec, fwd, bwd = r["rec"], r["fwd"], r["bwd"]
        ids = rec["vis_ids"]

        def per_gauss(a, w):
            out = np.zeros((n, w))
            out[ids] = np.asarray(a, np.float64).reshape(-1, w)
            return out

        vis = np.zeros(n, np.int8)
        vis[ids] = 1
        acc = oracle.project_backward(params, sc.cameras[r["view"]], st, vis, per_gauss(bwd["d_mean2d"], 2),
                                      per_gauss(bwd["d_conic"], 3), per_gauss(bwd["d_opacity"], 1)[:, 0],
                                      per_gauss(bwd["d_color"], 3), acc=acc)
        views.append(dict(
            vis_ids=ids.tolist(), proj_flag=[int(x) for x in rec["flag"]],
            mean2d=rec["mean2d"].tolist(), conic=rec["conic"].tolist(), opacity=rec["opacity"].tolist(),
            color=rec["color"].tolist(), depth=rec["depth"].tolist(), rect=rec["rect"].tolist(),
            n_tiles=rec["n_tiles"].tolist(), ranges=r["bins"]["ranges"].tolist(), vals=r["bins"]["vals"].tolist(),
            image_sum=fwd["image"].sum(axis=(1, 2)).tolist(), flagged_pixels=int(fwd["flag"].sum()),
            image_sum_err=fwd["err_C"].sum(axis=(1, 2)).tolist(),
            pixels=[dict(x=x, y=y, C=fwd["image"][:, y, x].tolist(), T=float(fwd["T_final"][y, x]),
                         n_contrib=int(fwd["n_contrib"][y, x]), flag=bool(fwd["flag"][y, x]),
                         err_C=fwd["err_C"][:, y, x].tolist(), err_T=float(fwd["err_T"][y, x]))
                    for x, y in SAMPLE_PIXELS],
            d_mean2d=bwd["d_mean2d"].tolist(), d_conic=bwd["d_conic"].tolist(), d_opacity=bwd["d_opacity"].tolist(),
            d_color=bwd["d_color"].tolist(), grad_bound=(2.0 * bwd["err"] + bwd["widen"]).tolist(),
            slot_flag=[bool(x) for x in bwd["slot_flag"]]))
    grads3d = {k: acc[k].tolist() for k in ("d_means", "d_log_scales", "d_quats", "d_opacity_logits", "d_sh")}
    return dict(views=views, grads3d=grads3d, grads3d_flag=[int(x) for x in acc["flag"]])


def main():
    import oracle
    sc = golden_scene()
    res = oracle_results(oracle, sc)
    res["source"] = ("written by tests/golden/make_golden.py from the CPU oracle (float64) on golden_scene(); "
                     "no page prints these values")
    with open(FIXTURE, "w") as f:
        json.dump(res, f, indent=None, separators=(",", ":"))
        f.write("\n")
    print("wrote", FIXTURE, os.path.getsize(FIXTURE), "bytes")


if __name__ == "__main__":
    main()
