"""The oracle against its stored results on the golden scene (tests/golden/tiny_two_views.json,
written by tests/golden/make_golden.py from the oracle itself): a regression record, so that a
change of the oracle's arithmetic shows here and is made on purpose (with the fixture written
again).  The oracle's correctness is pinned by the other oracle tests (closed forms, brute
force, finite differences); this file pins its stability."""
import json
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402

def close(now, stored, what):
    """Equal up to the summation order of the oracle's threads: 1e-12 relative, and 1e-12 of the
    array's largest magnitude absolute (components that cancel to near zero)."""
    a, b = np.asarray(stored, np.float64), np.asarray(now, np.float64)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12 * max(1e-300, float(np.abs(a).max(initial=0.0))),
                               err_msg=what)


INT_KEYS = ("vis_ids", "proj_flag", "rect", "n_tiles", "ranges", "vals", "slot_flag")
FLOAT_KEYS = ("mean2d", "conic", "opacity", "color", "depth", "image_sum", "image_sum_err", "d_mean2d", "d_conic",
              "d_opacity", "d_color", "grad_bound")


@pytest.fixture(scope="module")
def results(oracle_mod):
    stored = json.load(open(make_golden.FIXTURE))
    return stored, make_golden.oracle_results(oracle_mod, make_golden.golden_scene())


def test_golden_scene_shape(results):
    stored, now = results
    assert len(now["views"]) == 2
    for v in now["views"]:
        # the near-plane, behind-camera and off-frustum Gaussians are culled in both views
        assert not set(v["vis_ids"]) & {36, 37, 38, 39}
        assert 3 in v["vis_ids"] and 20 in v["vis_ids"]
        assert v["flagged_pixels"] == 0


def test_oracle_matches_its_stored_results(results):
    stored, now = results
    for a, b in zip(stored["views"], now["views"]):
        for k in INT_KEYS:
            assert a[k] == b[k], k
        for k in FLOAT_KEYS:
            close(b[k], a[k], k)
        for p, q in zip(a["pixels"], b["pixels"]):
            assert (p["x"], p["y"], p["n_contrib"], p["flag"]) == (q["x"], q["y"], q["n_contrib"], q["flag"])
            close(q["C"] + [q["T"]], p["C"] + [p["T"]], "pixel")
    for k, a in stored["grads3d"].items():
        close(now["grads3d"][k], a, k)
    assert stored["grads3d_flag"] == now["grads3d_flag"]
