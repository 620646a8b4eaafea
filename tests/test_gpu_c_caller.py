"""The hot path driven from plain C (tests/c/iteration_from_c.c: the C ABI and the HIP runtime's C
API, no Python or PyTorch in the process) on a seeded scene, its outputs checked against the
oracle like the other parity tests: projection end to end, bins, forward and backward stage by
stage on the GPU's own records.  Needs an MI355X."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import parity
from differentiable_raster_amd import scenes

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_DIR = os.path.join(ROOT, "differentiable_raster_amd")
ROCM = "/opt/rocm"


def _write_scene(path, sc):
    cam = sc.cameras[0]
    with open(path, "wb") as f:
        np.array([sc.n, cam.width, cam.height, sc.sh_degree], np.int32).tofile(f)
        np.concatenate([np.array([cam.fx, cam.fy, cam.cx, cam.cy], np.float32), cam.R.reshape(-1), cam.t,
                        cam.campos]).astype(np.float32).tofile(f)
        for a in (sc.means, sc.log_scales, sc.quats, sc.opacity_logits, sc.sh, sc.target[0]):
            np.ascontiguousarray(a, np.float32).tofile(f)


def _read_outputs(path, W, H):
    raw = open(path, "rb").read()
    pos = 0

    def take(dtype, count, shape=None):
        nonlocal pos
        a = np.frombuffer(raw, dtype, count, pos)
        pos += a.nbytes
        return a.reshape(shape) if shape else a

    vis = int(take(np.int32, 1)[0])
    m = int(take(np.int64, 1)[0])
    tiles = int(take(np.int32, 1)[0])
    out = dict(vis_count=vis, inst_count=m)
    out["vis_ids"] = take(np.int32, vis)
    out["mean2d"] = take(np.float32, 2 * vis, (vis, 2))
    out["conic_opacity"] = take(np.float32, 4 * vis, (vis, 4))
    out["color"] = take(np.float32, 3 * vis, (vis, 3))
    out["depth"] = take(np.float32, vis)
    out["rect"] = take(np.uint16, 4 * vis, (vis, 4)).astype(np.int32)
    out["n_tiles"] = take(np.int32, vis)
    bins = dict(ranges=take(np.int32, 2 * tiles, (tiles, 2)), tile_keys=take(np.uint32, m), vals=take(np.int32, m))
    img = take(np.float32, 3 * H * W, (3, H, W))
    T = take(np.float32, H * W, (H, W))
    nc = take(np.int32, H * W, (H, W))
    img_fused = take(np.float32, 3 * H * W, (3, H, W))
    grads = dict(d_mean2d=take(np.float32, 2 * vis, (vis, 2)), d_conic=take(np.float32, 3 * vis, (vis, 3)),
                 d_opacity=take(np.float32, vis), d_color=take(np.float32, 3 * vis, (vis, 3)))
    assert pos == len(raw)
    return out, bins, img, T, nc, img_fused, grads


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_iteration_driven_from_c(oracle_mod):
    oracle = oracle_mod
    sc = scenes.random_scene(700, 80, 56, seed=47, views=1, sh_degree=1, log_scale_mean=-2.5)
    st = sc.settings()
    cam = sc.cameras[0]
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "iteration_from_c")
        cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", f"{ROCM}/include",
               "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c", "iteration_from_c.c"), "-L", LIB_DIR,
               "-lgsmi", "-L", f"{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{LIB_DIR}", f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        scene_bin, out_bin = os.path.join(d, "scene.bin"), os.path.join(d, "out.bin")
        _write_scene(scene_bin, sc)
        print(f"[c caller] {sc.name}", flush=True)
        r = subprocess.run([exe, scene_bin, out_bin], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        print(r.stdout.strip(), flush=True)
        gpu, bins, img, T, nc, img_fused, grads = _read_outputs(out_bin, cam.width, cam.height)
    assert gpu["vis_count"] > 100
    parity.compare_projection(oracle, sc, cam, st, gpu)
    b = parity.compare_binning(oracle, cam, gpu, bins)
    rec = parity.gpu_records(gpu)
    f = parity.compare_forward(oracle, cam, st, rec, b["ranges"], b["vals"], img, T, nc)
    assert np.array_equal(img_fused.view(np.uint32), img.view(np.uint32)), "fused image differs from the forward's"
    dldc, dg = oracle.loss_grad_l1(f["image"], sc.target[0], 1.0, f["err_C"])
    parity.compare_backward(oracle, cam, st, rec, b["ranges"], b["vals"], dldc, grads, dg=dg, slots_rect=gpu["rect"])
