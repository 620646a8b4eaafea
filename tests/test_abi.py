"""The C-ABI library loads, exports every entry point its header declares, and rejects bad
arguments on the host before anything reaches the GPU (these calls never touch a device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsmi.h")


@pytest.fixture(scope="module")
def gs():
    from differentiable_raster_amd import gsmi
    if not os.path.exists(gsmi.LIB_PATH):
        from differentiable_raster_amd import build
        build.build()
    gsmi.load()
    return gsmi


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gs_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ["gs_project", "gs_bin_tiles", "gs_raster_fwd", "gs_raster_bwd", "gs_raster_fused",
                 "gs_fused_max_cap", "gs_loss_l1_grad", "gs_project_workspace_size", "gs_bin_workspace_size",
                 "gs_project_bwd", "gs_project_bwd_seen", "gs_adam_step_seen", "gs_raster_workspace_size", "gs_grad_encode", "gs_grad_decode",
                 "gs_grad_encode_workspace_size", "gs_compose", "gs_adam_step", "gs_adam_flush",
                 "gs_version", "gs_status_string", "gs_last_error", "gs_readback_create", "gs_readback_destroy"]:
        assert must in names, must


def test_library_exports_every_declared_symbol(gs):
    lib = ctypes.CDLL(gs.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings(gs):
    lib = gs.load()
    assert b"gfx950" in lib.gs_version()
    assert lib.gs_status_string(0) == b"ok"
    assert lib.gs_status_string(2) == b"capacity exceeded"


def test_fused_max_cap(gs):
    assert gs.gs_fused_max_cap() >= 256
    assert gs.load().gs_fused_max_cap(None) == 1


def test_workspace_queries(gs):
    assert gs.gs_project_workspace_size(1000, 4) > 0
    assert gs.gs_project_workspace_size(-1, 4) == 0
    assert gs.gs_bin_workspace_size(1000, 4, 128, 128, 5000) > gs.gs_bin_workspace_size(1000, 4, 128, 128, 10)
    assert gs.gs_bin_workspace_size(10, 0, 128, 128, 10) == 0


FAKE = 0x10000  # never dereferenced: validation fails before any device access


def cams(gs, V=1, w=64, h=48):
    from differentiable_raster_amd import scenes
    return gs.make_cameras([scenes.identity_camera(w, h) for _ in range(V)])


def params(gs, **kw):
    from differentiable_raster_amd import scenes
    s = scenes.RenderSettings(sh_degree=0)
    for k, v in kw.items():
        setattr(s, k, v)
    return gs.make_params(s)


def projected(gs, capacity=100, null=()):
    fields = {f: FAKE for f, _ in gs.gs_projected._fields_ if f != "capacity"}
    fields["readback"] = None  # a host object: a fake address would be dereferenced
    for f in null:
        fields[f] = None
    return gs.gs_projected(capacity, *[fields[f] for f, _ in gs.gs_projected._fields_ if f != "capacity"])


def test_project_bwd_rejects_bad_arguments(gs):
    lib = gs.load()
    g = gs.gs_gaussians(100, FAKE, FAKE, FAKE, FAKE, FAKE)
    c = cams(gs)
    p = params(gs)
    pr = projected(gs)
    g2 = gs.gs_grads2d(FAKE, FAKE, FAKE, FAKE)
    g3 = gs.gs_grads3d(FAKE, FAKE, FAKE, FAKE, FAKE)
    call = lambda g_, V, p_, pr_, a, b: lib.gs_project_bwd(g_, c, V, p_, pr_, a, b, None)
    assert call(None, 1, ctypes.byref(p), ctypes.byref(pr), ctypes.byref(g2), ctypes.byref(g3)) == 1
    assert call(ctypes.byref(g), 0, ctypes.byref(p), ctypes.byref(pr), ctypes.byref(g2), ctypes.byref(g3)) == 1
    assert call(ctypes.byref(g), 1, ctypes.byref(params(gs, sh_degree=5)), ctypes.byref(pr), ctypes.byref(g2),
                ctypes.byref(g3)) == 1
    assert call(ctypes.byref(g), 1, ctypes.byref(p), None, ctypes.byref(g2), ctypes.byref(g3)) == 1
    small = projected(gs, capacity=50)
    assert call(ctypes.byref(g), 1, ctypes.byref(p), ctypes.byref(small), ctypes.byref(g2), ctypes.byref(g3)) == 1
    assert call(ctypes.byref(g), 1, ctypes.byref(p), ctypes.byref(pr), None, ctypes.byref(g3)) == 1
    assert call(ctypes.byref(g), 1, ctypes.byref(p), ctypes.byref(pr), ctypes.byref(gs.gs_grads2d(FAKE, FAKE, None, FAKE)),
                ctypes.byref(g3)) == 1
    assert call(ctypes.byref(g), 1, ctypes.byref(p), ctypes.byref(pr), ctypes.byref(g2), None) == 1
    assert call(ctypes.byref(g), 1, ctypes.byref(p), ctypes.byref(pr), ctypes.byref(g2),
                ctypes.byref(gs.gs_grads3d(FAKE, FAKE, FAKE, FAKE, None))) == 1
    assert b"null" in lib.gs_last_error()
    g_null = gs.gs_gaussians(100, FAKE, FAKE, None, FAKE, FAKE)
    assert call(ctypes.byref(g_null), 1, ctypes.byref(p), ctypes.byref(pr), ctypes.byref(g2), ctypes.byref(g3)) == 1
    # the seen-flag variant: the same checks, and the flags must be given
    seen = lambda g_, s: lib.gs_project_bwd_seen(g_, c, 1, ctypes.byref(p), ctypes.byref(pr), ctypes.byref(g2),
                                                 ctypes.byref(g3), s, None)
    assert seen(ctypes.byref(g), None) == 1
    assert b"seen" in lib.gs_last_error()
    assert seen(ctypes.byref(g_null), FAKE) == 1
    assert seen(None, FAKE) == 1


def test_grad_codec_rejects_bad_arguments(gs):
    lib = gs.load()
    g2 = gs.gs_grads2d(FAKE, FAKE, FAKE, FAKE)
    need = lib.gs_grad_encode_workspace_size(1000, 2)
    assert need > 0 and lib.gs_grad_encode_workspace_size(1000, 0) == 0
    enc = lambda V, cap, a, b, c, gr, ws, wsb: lib.gs_grad_encode(V, cap, a, FAKE, gr, b, c, FAKE, ws, wsb, None)
    assert enc(0, 1000, FAKE, FAKE, FAKE, ctypes.byref(g2), FAKE, need) == 1
    assert enc(2, -1, FAKE, FAKE, FAKE, ctypes.byref(g2), FAKE, need) == 1
    assert enc(2, 1000, None, FAKE, FAKE, ctypes.byref(g2), FAKE, need) == 1
    assert enc(2, 1000, FAKE, None, FAKE, ctypes.byref(g2), FAKE, need) == 1
    assert enc(2, 1000, FAKE, FAKE, FAKE, ctypes.byref(gs.gs_grads2d(FAKE, None, FAKE, FAKE)), FAKE, need) == 1
    assert enc(2, 1000, FAKE, FAKE, FAKE, None, FAKE, need) == 1
    assert enc(2, 1000, FAKE, FAKE, FAKE, ctypes.byref(g2), FAKE, need - 1) == 2
    assert enc(2, 1000, FAKE, FAKE, FAKE, ctypes.byref(g2), FAKE + 16, need) == 1  # not 256-byte aligned
    assert enc(16, 1 << 27, FAKE, FAKE, FAKE, ctypes.byref(g2), FAKE, need) == 1  # records past 2^31
    dec = lambda V, n, m, o: lib.gs_grad_decode(V, n, m, FAKE, FAKE, FAKE, o, None)
    assert dec(0, 10, 10, ctypes.byref(g2)) == 1
    assert dec(1, -1, 10, ctypes.byref(g2)) == 1
    assert dec(1, 10, -1, ctypes.byref(g2)) == 1
    assert dec(1, 10, 10, None) == 1
    assert dec(1, 10, 10, ctypes.byref(gs.gs_grads2d(FAKE, FAKE, FAKE, None))) == 1
    assert lib.gs_grad_decode(1, 10, 10, None, FAKE, FAKE, ctypes.byref(g2), None) == 1


def test_compose_rejects_bad_arguments(gs):
    lib = gs.load()
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    bg = (ctypes.c_float * 3)(0.0, 0.0, 0.0)
    call = lambda P, V, W, H, c, t, b, img: lib.gs_compose(P, V, W, H, c, t, b, img, None, None)
    assert call(0, 1, 8, 8, arr(FAKE), arr(FAKE), bg, FAKE) == 1
    assert call(17, 1, 8, 8, arr(*[FAKE] * 17), arr(*[FAKE] * 17), bg, FAKE) == 1
    assert call(1, 0, 8, 8, arr(FAKE), arr(FAKE), bg, FAKE) == 1
    assert call(1, 1, 0, 8, arr(FAKE), arr(FAKE), bg, FAKE) == 1
    assert call(2, 1, 8, 8, arr(FAKE, None), arr(FAKE, FAKE), bg, FAKE) == 1
    assert call(1, 1, 8, 8, None, arr(FAKE), bg, FAKE) == 1
    assert call(1, 1, 8, 8, arr(FAKE), arr(FAKE), None, FAKE) == 1
    assert call(1, 1, 8, 8, arr(FAKE), arr(FAKE), bg, None) == 1
    assert call(1, 1, 8, 8, arr(FAKE), arr(FAKE), (ctypes.c_float * 3)(float("nan"), 0.0, 0.0), FAKE) == 1


def test_adam_rejects_bad_arguments(gs):
    lib = gs.load()
    grp = lambda **k: gs.gs_adam_group(**{**dict(param=FAKE, grad=FAKE, m=FAKE, v=FAKE, rows=3, lr=0.01), **k})
    groups = (gs.gs_adam_group * 2)(grp(), grp(rows=48))
    hp = gs.gs_adam_params(0.9, 0.999, 1e-15)
    step = lambda n, g, ng, h, t, last=FAKE, act=None, na=0: lib.gs_adam_step(n, g, ng, h, t, last, act, na, None)
    assert step(-1, groups, 2, ctypes.byref(hp), 1) == 1
    assert step(10, None, 2, ctypes.byref(hp), 1) == 1
    assert step(10, groups, 0, ctypes.byref(hp), 1) == 1
    assert step(10, groups, 9, ctypes.byref(hp), 1) == 1
    assert step(10, groups, 2, None, 1) == 1
    assert step(10, groups, 2, ctypes.byref(gs.gs_adam_params(1.0, 0.999, 1e-15)), 1) == 1
    assert step(10, groups, 2, ctypes.byref(gs.gs_adam_params(0.9, 0.999, 0.0)), 1) == 1
    assert step(10, groups, 2, ctypes.byref(hp), 0) == 1
    assert step(10, (gs.gs_adam_group * 1)(grp(m=None)), 1, ctypes.byref(hp), 1) == 1
    assert step(10, (gs.gs_adam_group * 1)(grp(rows=0)), 1, ctypes.byref(hp), 1) == 1
    assert step(10, (gs.gs_adam_group * 1)(grp(lr=float("inf"))), 1, ctypes.byref(hp), 1) == 1
    assert step(10, groups, 2, ctypes.byref(hp), 1, FAKE, FAKE, -1) == 1
    assert lib.gs_adam_flush(10, groups, 2, ctypes.byref(hp), 1, None, None) == 1
    step_seen = lambda n, last, seen, t=1: lib.gs_adam_step_seen(n, groups, 2, ctypes.byref(hp), t, last, seen, None)
    assert step_seen(10, None, FAKE) == 1
    assert step_seen(10, FAKE, None) == 1
    assert step_seen(-1, FAKE, FAKE) == 1
    assert step_seen(10, FAKE, FAKE, t=0) == 1


def test_project_rejects_bad_arguments(gs):
    lib = gs.load()
    g = gs.gs_gaussians(100, FAKE, FAKE, FAKE, FAKE, FAKE)
    c = cams(gs)
    p = params(gs)
    out = projected(gs)
    ws_ok = gs.gs_project_workspace_size(100, 1)
    call = lambda g_, c_, V, p_, o_, ws, nbytes: lib.gs_project(g_, c_, V, p_, o_, ws, nbytes, None)
    assert call(None, c, 1, ctypes.byref(p), ctypes.byref(out), FAKE, ws_ok) == 1
    assert call(ctypes.byref(g), None, 1, ctypes.byref(p), ctypes.byref(out), FAKE, ws_ok) == 1
    assert call(ctypes.byref(g), c, 0, ctypes.byref(p), ctypes.byref(out), FAKE, ws_ok) == 1
    assert call(ctypes.byref(g), c, 17, ctypes.byref(p), ctypes.byref(out), FAKE, ws_ok) == 1
    bad = params(gs, sh_degree=4)
    assert call(ctypes.byref(g), c, 1, ctypes.byref(bad), ctypes.byref(out), FAKE, ws_ok) == 1
    bad = params(gs, alpha_max=1.0)
    assert call(ctypes.byref(g), c, 1, ctypes.byref(bad), ctypes.byref(out), FAKE, ws_ok) == 1
    # depth keys need positive depths; non-finite constants are refused
    for kw in (dict(znear=-0.1), dict(znear=float("nan")), dict(znear=float("inf")), dict(eps2d=float("inf")),
               dict(bg=(0.0, float("nan"), 0.0))):
        bad = params(gs, **kw)
        assert call(ctypes.byref(g), c, 1, ctypes.byref(bad), ctypes.byref(out), FAKE, ws_ok) == 1, kw
    ok = params(gs, znear=0.0)
    assert call(ctypes.byref(g), c, 1, ctypes.byref(ok), ctypes.byref(out), FAKE, ws_ok - 1) == 2  # past the checks
    small = projected(gs, capacity=50)
    assert call(ctypes.byref(g), c, 1, ctypes.byref(p), ctypes.byref(small), FAKE, ws_ok) == 1
    assert b"capacity" in lib.gs_last_error()
    # the per-field copies of centre, conic/opacity and colour are optional: past the checks
    lean = projected(gs, null=("mean2d", "conic_opacity", "color"))
    assert call(ctypes.byref(g), c, 1, ctypes.byref(p), ctypes.byref(lean), FAKE, ws_ok - 1) == 2
    for f in ("vis_ids", "depth", "tile_rect", "n_tiles", "inst_base", "raster_rec"):
        nulls = projected(gs, null=(f,))
        assert call(ctypes.byref(g), c, 1, ctypes.byref(p), ctypes.byref(nulls), FAKE, ws_ok) == 1
    skew = projected(gs)
    skew.raster_rec = FAKE + 16
    assert call(ctypes.byref(g), c, 1, ctypes.byref(p), ctypes.byref(skew), FAKE, ws_ok) == 1
    assert b"aligned" in lib.gs_last_error()
    g_null = gs.gs_gaussians(100, FAKE, None, FAKE, FAKE, FAKE)
    assert call(ctypes.byref(g_null), c, 1, ctypes.byref(p), ctypes.byref(out), FAKE, ws_ok) == 1
    g_big = gs.gs_gaussians(1 << 28, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert call(ctypes.byref(g_big), c, 1, ctypes.byref(p), ctypes.byref(out), FAKE, ws_ok) == 1
    # workspace too small -> capacity error, nothing launched
    assert call(ctypes.byref(g), c, 1, ctypes.byref(p), ctypes.byref(out), FAKE, ws_ok - 1) == 2
    assert call(ctypes.byref(g), c, 1, ctypes.byref(p), ctypes.byref(out), None, ws_ok) == 2
    # views of different image sizes
    from differentiable_raster_amd import scenes
    mixed = gs.make_cameras([scenes.identity_camera(64, 48), scenes.identity_camera(32, 48)])
    assert call(ctypes.byref(g), mixed, 2, ctypes.byref(p), ctypes.byref(out), FAKE, ws_ok) == 1


def test_bin_and_raster_reject_bad_arguments(gs):
    lib = gs.load()
    c = cams(gs)
    p = params(gs)
    proj = projected(gs)
    bins = gs.gs_bins(1000, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    info = gs.gs_bin_info()
    req = ctypes.c_int64()
    ws = gs.gs_bin_workspace_size(100, 1, 64, 48, 1000)
    assert lib.gs_bin_tiles(c, ctypes.byref(proj), 1, ctypes.byref(p), None, ctypes.byref(info), ctypes.byref(req),
                            FAKE, ws, None) == 1
    assert lib.gs_bin_tiles(c, ctypes.byref(proj), 1, ctypes.byref(p), ctypes.byref(bins), None, ctypes.byref(req),
                            FAKE, ws, None) == 1
    assert lib.gs_bin_tiles(c, ctypes.byref(proj), 1, ctypes.byref(p), ctypes.byref(bins), ctypes.byref(info),
                            ctypes.byref(req), FAKE, ws - 1, None) == 2
    capped = params(gs, tile_cap=64)
    nocap = gs.gs_bins(1000, 10, FAKE, FAKE, FAKE, None, None, None, None)
    assert lib.gs_bin_tiles(c, ctypes.byref(proj), 1, ctypes.byref(capped), ctypes.byref(nocap), ctypes.byref(info),
                            ctypes.byref(req), FAKE, ws, None) == 1
    # the cap's scores need the conic and opacity: from conic_opacity, else from the packed records
    for nulls, code in ((("conic_opacity",), 2), (("raster_rec",), 2), (("conic_opacity", "raster_rec"), 1)):
        pr = projected(gs, null=nulls)
        assert lib.gs_bin_tiles(c, ctypes.byref(pr), 1, ctypes.byref(capped), ctypes.byref(bins), ctypes.byref(info),
                                ctypes.byref(req), FAKE, ws - 1, None) == code, nulls
    lean = projected(gs, null=("conic_opacity", "raster_rec"))
    assert lib.gs_bin_tiles(c, ctypes.byref(lean), 1, ctypes.byref(p), ctypes.byref(bins), ctypes.byref(info),
                            ctypes.byref(req), FAKE, ws - 1, None) == 2  # uncapped: neither is read
    neg = params(gs, tile_cap=-1)
    assert lib.gs_bin_tiles(c, ctypes.byref(proj), 1, ctypes.byref(neg), ctypes.byref(bins), ctypes.byref(info),
                            ctypes.byref(req), FAKE, ws, None) == 1
    # a failed gs_bin_tiles marks the bins unusable, and the raster calls refuse them
    assert bins.count == -1
    grads = gs.gs_grads2d(FAKE, FAKE, FAKE, FAKE)
    assert lib.gs_raster_fwd(c, ctypes.byref(proj), ctypes.byref(bins), 1, ctypes.byref(p), 0, FAKE, FAKE, FAKE, None,
                             None) == 1
    bins.count = 10
    assert lib.gs_raster_fwd(c, ctypes.byref(proj), None, 1, ctypes.byref(p), 0, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.gs_raster_fwd(c, ctypes.byref(proj), ctypes.byref(bins), 1, ctypes.byref(p), 0, None, FAKE, FAKE, None,
                             None) == 1
    rws = gs.gs_raster_workspace_size(1000)
    assert rws >= 1000 * 36
    assert lib.gs_raster_bwd(c, ctypes.byref(proj), ctypes.byref(bins), 1, ctypes.byref(p), 0, FAKE, FAKE, FAKE, None,
                             ctypes.byref(grads), FAKE, rws, None) == 1
    bad_grads = gs.gs_grads2d(FAKE, None, FAKE, FAKE)
    assert lib.gs_raster_bwd(c, ctypes.byref(proj), ctypes.byref(bins), 1, ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE,
                             ctypes.byref(bad_grads), FAKE, rws, None) == 1
    # partial-record workspace too small for bins->count instances
    assert lib.gs_raster_bwd(c, ctypes.byref(proj), ctypes.byref(bins), 1, ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE,
                             ctypes.byref(grads), FAKE, 10 * 36 - 1, None) == 2
    assert lib.gs_raster_fused(c, ctypes.byref(proj), ctypes.byref(bins), 1, ctypes.byref(p), 0, 7, FAKE,
                               ctypes.c_float(1.0), None, None, ctypes.byref(grads), None, FAKE, rws, None) == 1
    assert lib.gs_raster_fused(c, ctypes.byref(proj), ctypes.byref(bins), 1, ctypes.byref(p), 0, 0, None,
                               ctypes.c_float(1.0), None, None, ctypes.byref(grads), None, FAKE, rws, None) == 1
    assert lib.gs_raster_fused(c, ctypes.byref(proj), ctypes.byref(bins), 1, ctypes.byref(p), 0, 0, FAKE,
                               ctypes.c_float(1.0), None, None, ctypes.byref(grads), None, None, 0, None) == 2
    assert lib.gs_loss_l1_grad(0, 64, 48, FAKE, FAKE, ctypes.c_float(1.0), FAKE, None, None) == 1
    assert lib.gs_loss_l1_grad(1, 64, 48, None, FAKE, ctypes.c_float(1.0), FAKE, None, None) == 1


def test_product_path_imports_no_oracle():
    """The binding and the pipeline never import the oracle (it is test infrastructure)."""
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle|from\s+\.\.?\s*import\s+oracle)|oracle[/.]|liboracle",
                     re.M)
    for f in ["gsmi.py", "pipeline.py", "scenes.py", "build.py", "__init__.py"]:
        src = open(os.path.join(ROOT, "differentiable_raster_amd", f)).read()
        assert not pat.search(src), f
    for f in os.listdir(os.path.join(ROOT, "differentiable_raster_amd", "csrc")):
        src = open(os.path.join(ROOT, "differentiable_raster_amd", "csrc", f)).read()
        assert "oracle" not in src.lower(), f


def test_readback_create_rejects_null(gs):
    assert gs.load().gs_readback_create(None) == 1
    gs.load().gs_readback_destroy(None)  # ignored


def test_project_noalloc_rejects_inputs_beyond_its_scratch(gs):
    """gs_project_noalloc refuses, on the host, inputs whose projection workspace exceeds its
    static 16 MiB scratch (nothing is launched, so the fake pointers are never touched)."""
    lib = gs.load()
    assert gs.gs_project_noalloc_max_bytes() == 16 << 20
    c = cams(gs, V=4)
    p = params(gs)
    n_fit = 6_000_000
    assert gs.gs_project_workspace_size(n_fit, 4) <= 16 << 20 < gs.gs_project_workspace_size(8_000_000, 4)
    g_big = gs.gs_gaussians(8_000_000, FAKE, FAKE, FAKE, FAKE, FAKE)
    out = projected(gs, capacity=8_000_000)
    assert lib.gs_project_noalloc(ctypes.byref(g_big), c, 4, ctypes.byref(p), ctypes.byref(out), None) == 2
    assert b"static scratch" in lib.gs_last_error()
    assert lib.gs_project_noalloc(None, c, 4, ctypes.byref(p), ctypes.byref(out), None) == 1


def test_check_bins_rejects_bad_arguments(gs):
    """gs_check_bins validates its arguments on the host before touching the device."""
    lib = gs.load()
    c = cams(gs)
    p = params(gs)
    pr = projected(gs)
    viol = (ctypes.c_int64 * gs.GS_CHECK_KINDS)()
    b = gs.gs_bins(100, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert lib.gs_check_bins(None, ctypes.byref(pr), 1, ctypes.byref(p), ctypes.byref(b), viol, None) == 1
    assert lib.gs_check_bins(c, None, 1, ctypes.byref(p), ctypes.byref(b), viol, None) == 1
    assert lib.gs_check_bins(c, ctypes.byref(pr), 1, ctypes.byref(p), None, viol, None) == 1
    assert lib.gs_check_bins(c, ctypes.byref(pr), 1, ctypes.byref(p), ctypes.byref(b), None, None) == 1
    failed = gs.gs_bins(100, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert lib.gs_check_bins(c, ctypes.byref(pr), 1, ctypes.byref(p), ctypes.byref(failed), viol, None) == 1
    assert b"successful" in lib.gs_last_error()
    capped = params(gs, tile_cap=4)
    nocap = gs.gs_bins(100, 10, FAKE, FAKE, FAKE, None, None, None, None)
    assert lib.gs_check_bins(c, ctypes.byref(pr), 1, ctypes.byref(capped), ctypes.byref(nocap), viol, None) == 1
