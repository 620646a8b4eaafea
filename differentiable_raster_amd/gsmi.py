"""Thin ctypes binding of libgsmi.so (include/gsmi.h), with the same entry-point names.

Only argument marshalling happens here: every step of the hot path runs in the HIP library.
PyTorch supplies device memory (tensors) and the stream (torch's current HIP stream).
Importing this module loads torch first, so that the library binds to the HIP runtime torch
already loaded, and then loads the library; a missing library raises immediately.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgsmi.so")

GS_MAX_VIEWS = 16
GS_TILE = 16
GS_LOSS_L1 = 0
GS_LOSS_EXTERNAL = 1
STATUS = {0: "GS_OK", 1: "GS_ERR_INVALID_ARGUMENT", 2: "GS_ERR_CAPACITY", 3: "GS_ERR_UNSUPPORTED",
          4: "GS_ERR_HIP", 5: "GS_ERR_INTERNAL"}


class GsError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {message}")
        self.status = status


class gs_camera(ctypes.Structure):
    _fields_ = [("width", ctypes.c_int32), ("height", ctypes.c_int32),
                ("fx", ctypes.c_float), ("fy", ctypes.c_float), ("cx", ctypes.c_float), ("cy", ctypes.c_float),
                ("R", ctypes.c_float * 9), ("t", ctypes.c_float * 3), ("campos", ctypes.c_float * 3)]


class gs_render_params(ctypes.Structure):
    _fields_ = [("znear", ctypes.c_float), ("eps2d", ctypes.c_float), ("alpha_min", ctypes.c_float),
                ("alpha_max", ctypes.c_float), ("t_min", ctypes.c_float), ("bg", ctypes.c_float * 3),
                ("sh_degree", ctypes.c_int32), ("tile_cap", ctypes.c_int32)]


class gs_gaussians(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("means", ctypes.c_void_p), ("log_scales", ctypes.c_void_p),
                ("quats", ctypes.c_void_p), ("opacity_logits", ctypes.c_void_p), ("sh", ctypes.c_void_p)]


class gs_projected(ctypes.Structure):
    _fields_ = [("capacity", ctypes.c_int32), ("vis_count", ctypes.c_void_p), ("inst_count", ctypes.c_void_p),
                ("vis_ids", ctypes.c_void_p), ("mean2d", ctypes.c_void_p), ("conic_opacity", ctypes.c_void_p),
                ("color", ctypes.c_void_p), ("depth", ctypes.c_void_p), ("tile_rect", ctypes.c_void_p),
                ("n_tiles", ctypes.c_void_p), ("inst_base", ctypes.c_void_p), ("raster_rec", ctypes.c_void_p),
                ("readback", ctypes.c_void_p)]


class gs_bins(ctypes.Structure):
    _fields_ = [("capacity", ctypes.c_int64), ("count", ctypes.c_int64), ("tile_keys", ctypes.c_void_p),
                ("vals", ctypes.c_void_p), ("ranges", ctypes.c_void_p), ("vals_capped", ctypes.c_void_p),
                ("ranges_capped", ctypes.c_void_p), ("num_capped", ctypes.c_void_p), ("tile_order", ctypes.c_void_p)]


class gs_bin_info(ctypes.Structure):
    _fields_ = [("vis_count", ctypes.c_int32 * GS_MAX_VIEWS), ("view_offset", ctypes.c_int64 * (GS_MAX_VIEWS + 1)),
                ("num_instances", ctypes.c_int64), ("num_instances_capped", ctypes.c_int64)]


class gs_grads2d(ctypes.Structure):
    _fields_ = [("d_mean2d", ctypes.c_void_p), ("d_conic", ctypes.c_void_p), ("d_opacity", ctypes.c_void_p),
                ("d_color", ctypes.c_void_p)]


class gs_grads3d(ctypes.Structure):
    _fields_ = [("d_means", ctypes.c_void_p), ("d_log_scales", ctypes.c_void_p), ("d_quats", ctypes.c_void_p),
                ("d_opacity_logits", ctypes.c_void_p), ("d_sh", ctypes.c_void_p)]


class gs_adam_group(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("rows", ctypes.c_int32), ("lr", ctypes.c_float)]


class gs_adam_params(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float)]


_P = ctypes.POINTER
_SIGS = {
    "gs_version": (ctypes.c_char_p, []),
    "gs_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gs_last_error": (ctypes.c_char_p, []),
    "gs_readback_create": (ctypes.c_int, [_P(ctypes.c_void_p)]),
    "gs_readback_destroy": (None, [ctypes.c_void_p]),
    "gs_project_workspace_size": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "gs_project": (ctypes.c_int, [_P(gs_gaussians), _P(gs_camera), ctypes.c_int32, _P(gs_render_params),
                                  _P(gs_projected), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "gs_project_noalloc": (ctypes.c_int, [_P(gs_gaussians), _P(gs_camera), ctypes.c_int32, _P(gs_render_params),
                                          _P(gs_projected), ctypes.c_void_p]),
    "gs_project_noalloc_max_bytes": (ctypes.c_size_t, []),
    "gs_bin_workspace_size": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int64]),
    "gs_bin_tiles": (ctypes.c_int, [_P(gs_camera), _P(gs_projected), ctypes.c_int32, _P(gs_render_params),
                                    _P(gs_bins), _P(gs_bin_info), _P(ctypes.c_int64), ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]),
    "gs_raster_fwd": (ctypes.c_int, [_P(gs_camera), _P(gs_projected), _P(gs_bins), ctypes.c_int32,
                                     _P(gs_render_params), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "gs_loss_l1_grad": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]),
    "gs_raster_bwd": (ctypes.c_int, [_P(gs_camera), _P(gs_projected), _P(gs_bins), ctypes.c_int32,
                                     _P(gs_render_params), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, _P(gs_grads2d), ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]),
    "gs_raster_fused": (ctypes.c_int, [_P(gs_camera), _P(gs_projected), _P(gs_bins), ctypes.c_int32,
                                       _P(gs_render_params), ctypes.c_int32, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, _P(gs_grads2d),
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "gs_raster_workspace_size": (ctypes.c_size_t, [ctypes.c_int64]),
    "gs_project_bwd": (ctypes.c_int, [_P(gs_gaussians), _P(gs_camera), ctypes.c_int32, _P(gs_render_params),
                                      _P(gs_projected), _P(gs_grads2d), _P(gs_grads3d), ctypes.c_void_p]),
    "gs_project_bwd_seen": (ctypes.c_int, [_P(gs_gaussians), _P(gs_camera), ctypes.c_int32, _P(gs_render_params),
                                           _P(gs_projected), _P(gs_grads2d), _P(gs_grads3d), ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "gs_fused_max_cap": (ctypes.c_int, [_P(ctypes.c_int32)]),
    "gs_check_bins": (ctypes.c_int, [_P(gs_camera), _P(gs_projected), ctypes.c_int32, _P(gs_render_params),
                                     _P(gs_bins), _P(ctypes.c_int64), ctypes.c_void_p]),
    "gs_grad_encode_workspace_size": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "gs_grad_encode": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                      _P(gs_grads2d), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "gs_grad_decode": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, _P(gs_grads2d), ctypes.c_void_p]),
    "gs_compose": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  _P(ctypes.c_void_p), _P(ctypes.c_void_p), _P(ctypes.c_float), ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]),
    "gs_adam_step": (ctypes.c_int, [ctypes.c_int32, _P(gs_adam_group), ctypes.c_int32, _P(gs_adam_params),
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_void_p]),
    "gs_adam_step_seen": (ctypes.c_int, [ctypes.c_int32, _P(gs_adam_group), ctypes.c_int32, _P(gs_adam_params),
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "gs_adam_flush": (ctypes.c_int, [ctypes.c_int32, _P(gs_adam_group), ctypes.c_int32, _P(gs_adam_params),
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libgsmi.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} is not built; run __graft_entry__.build() or "
                                    f"python differentiable_raster_amd/build.py")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        if not t.is_cuda:
            raise ValueError("device tensor expected")
        if not t.is_contiguous():
            raise ValueError("contiguous tensor expected")
        return t.data_ptr()
    return int(t)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, where: str):
    if status != 0:
        raise GsError(status, where, load().gs_last_error().decode())


def make_cameras(cams) -> ctypes.Array:
    arr = (gs_camera * len(cams))()
    for i, c in enumerate(cams):
        arr[i].width, arr[i].height = int(c.width), int(c.height)
        arr[i].fx, arr[i].fy, arr[i].cx, arr[i].cy = float(c.fx), float(c.fy), float(c.cx), float(c.cy)
        R = [float(x) for x in c.R.reshape(9)]
        t = [float(x) for x in c.t.reshape(3)]
        cp = [float(x) for x in c.campos.reshape(3)]
        for k in range(9):
            arr[i].R[k] = R[k]
        for k in range(3):
            arr[i].t[k] = t[k]
            arr[i].campos[k] = cp[k]
    return arr


def make_params(s) -> gs_render_params:
    p = gs_render_params()
    p.znear, p.eps2d = s.znear, s.eps2d
    p.alpha_min, p.alpha_max, p.t_min = s.alpha_min, s.alpha_max, s.t_min
    for k in range(3):
        p.bg[k] = s.bg[k]
    p.sh_degree, p.tile_cap = int(s.sh_degree), int(s.tile_cap)
    return p


# ---------------------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------------
def gs_version() -> str:
    return load().gs_version().decode()


def gs_readback_create() -> int:
    """A pinned host count buffer for gs_projected.readback (an opaque handle)."""
    h = ctypes.c_void_p()
    _check(load().gs_readback_create(ctypes.byref(h)), "gs_readback_create")
    return int(h.value)


def gs_readback_destroy(handle) -> None:
    load().gs_readback_destroy(handle)


def gs_project_workspace_size(n: int, V: int) -> int:
    return int(load().gs_project_workspace_size(n, V))


def gs_raster_workspace_size(instance_capacity: int) -> int:
    return int(load().gs_raster_workspace_size(instance_capacity))


def gs_bin_workspace_size(n: int, V: int, width: int, height: int, instance_capacity: int) -> int:
    return int(load().gs_bin_workspace_size(n, V, width, height, instance_capacity))


GS_CHECK_KINDS = 8
GS_CHECK_NAMES = ("range", "key", "slot", "rect", "order", "count", "cap", "slot_record")


def gs_check_bins(cams, proj: gs_projected, V: int, params: gs_render_params, bins: gs_bins, stream=None):
    """GS_CHECK: (status, {kind: violations}) of the device validation of the tile lists."""
    out = (ctypes.c_int64 * GS_CHECK_KINDS)()
    st = load().gs_check_bins(cams, ctypes.byref(proj), V, ctypes.byref(params), ctypes.byref(bins), out,
                              _stream(stream))
    if st not in (0, 5):  # GS_ERR_INTERNAL reports violations
        _check(st, "gs_check_bins")
    return st, dict(zip(GS_CHECK_NAMES, [int(x) for x in out]))


def gs_fused_max_cap() -> int:
    k = ctypes.c_int32()
    _check(load().gs_fused_max_cap(ctypes.byref(k)), "gs_fused_max_cap")
    return k.value


def gs_project(g: gs_gaussians, cams, V: int, params: gs_render_params, out: gs_projected, ws, stream=None):
    _check(load().gs_project(ctypes.byref(g), cams, V, ctypes.byref(params), ctypes.byref(out), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "gs_project")


def gs_project_noalloc(g: gs_gaussians, cams, V: int, params: gs_render_params, out: gs_projected, stream=None):
    _check(load().gs_project_noalloc(ctypes.byref(g), cams, V, ctypes.byref(params), ctypes.byref(out),
                                     _stream(stream)), "gs_project_noalloc")


def gs_project_noalloc_max_bytes() -> int:
    return int(load().gs_project_noalloc_max_bytes())


def gs_project_bwd(g: gs_gaussians, cams, V: int, params: gs_render_params, proj: gs_projected,
                   grads2d: gs_grads2d, out: gs_grads3d, stream=None):
    _check(load().gs_project_bwd(ctypes.byref(g), cams, V, ctypes.byref(params), ctypes.byref(proj),
                                 ctypes.byref(grads2d), ctypes.byref(out), _stream(stream)), "gs_project_bwd")


def gs_project_bwd_seen(g: gs_gaussians, cams, V: int, params: gs_render_params, proj: gs_projected,
                        grads2d: gs_grads2d, out: gs_grads3d, seen, stream=None):
    """seen: device uint8 [n], written."""
    _check(load().gs_project_bwd_seen(ctypes.byref(g), cams, V, ctypes.byref(params), ctypes.byref(proj),
                                      ctypes.byref(grads2d), ctypes.byref(out), _ptr(seen), _stream(stream)),
           "gs_project_bwd_seen")


def gs_bin_tiles(cams, proj: gs_projected, V: int, params: gs_render_params, bins: gs_bins, ws, stream=None):
    """Returns (status, gs_bin_info, required); raises on any error except GS_ERR_CAPACITY."""
    info = gs_bin_info()
    req = ctypes.c_int64(0)
    st = load().gs_bin_tiles(cams, ctypes.byref(proj), V, ctypes.byref(params), ctypes.byref(bins),
                             ctypes.byref(info), ctypes.byref(req), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream))
    if st not in (0, 2):
        _check(st, "gs_bin_tiles")
    return st, info, req.value


def gs_raster_fwd(cams, proj, bins, V, params, use_capped, image, t_final, n_contrib, counters=None, stream=None):
    _check(load().gs_raster_fwd(cams, ctypes.byref(proj), ctypes.byref(bins), V, ctypes.byref(params),
                                int(use_capped), _ptr(image), _ptr(t_final), _ptr(n_contrib), _ptr(counters),
                                _stream(stream)), "gs_raster_fwd")


def gs_loss_l1_grad(V, width, height, image, target, scale, dl, loss_sum=None, stream=None):
    _check(load().gs_loss_l1_grad(V, width, height, _ptr(image), _ptr(target), float(scale), _ptr(dl),
                                  _ptr(loss_sum), _stream(stream)), "gs_loss_l1_grad")


def gs_raster_bwd(cams, proj, bins, V, params, use_capped, image, t_final, n_contrib, dl, grads: gs_grads2d,
                  ws, stream=None):
    _check(load().gs_raster_bwd(cams, ctypes.byref(proj), ctypes.byref(bins), V, ctypes.byref(params),
                                int(use_capped), _ptr(image), _ptr(t_final), _ptr(n_contrib), _ptr(dl),
                                ctypes.byref(grads), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "gs_raster_bwd")


def gs_raster_fused(cams, proj, bins, V, params, use_capped, mode, target_or_dl, scale, image, loss_sum,
                    grads: gs_grads2d, ws, counters=None, stream=None):
    _check(load().gs_raster_fused(cams, ctypes.byref(proj), ctypes.byref(bins), V, ctypes.byref(params),
                                  int(use_capped), int(mode), _ptr(target_or_dl), float(scale), _ptr(image),
                                  _ptr(loss_sum), ctypes.byref(grads), _ptr(counters), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)),
           "gs_raster_fused")


def gs_grad_encode_workspace_size(capacity: int, V: int) -> int:
    return int(load().gs_grad_encode_workspace_size(capacity, V))


def gs_grad_encode(V, capacity, vis_count, vis_ids, grads: gs_grads2d, keys, records, view_offset, ws, stream=None):
    _check(load().gs_grad_encode(V, capacity, _ptr(vis_count), _ptr(vis_ids), ctypes.byref(grads), _ptr(keys),
                                 _ptr(records), _ptr(view_offset), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "gs_grad_encode")


def gs_grad_decode(V, n_owner, max_records, view_offset, keys, records, owner: gs_grads2d, stream=None):
    _check(load().gs_grad_decode(V, n_owner, int(max_records), _ptr(view_offset), _ptr(keys), _ptr(records),
                                 ctypes.byref(owner), _stream(stream)), "gs_grad_decode")


def gs_compose(V, width, height, colors, t_finals, bg, image, t_out=None, stream=None):
    """colors / t_finals: sequences of device tensors, front to back."""
    P = len(colors)
    c_arr = (ctypes.c_void_p * P)(*[_ptr(c) for c in colors])
    t_arr = (ctypes.c_void_p * P)(*[_ptr(t) for t in t_finals])
    bg_arr = (ctypes.c_float * 3)(*[float(x) for x in bg])
    _check(load().gs_compose(P, V, width, height, c_arr, t_arr, bg_arr, _ptr(image), _ptr(t_out), _stream(stream)),
           "gs_compose")


def gs_adam_step(n, groups, hp: gs_adam_params, t, last_step=None, active=None, n_active=0, stream=None):
    """groups: a ctypes array of gs_adam_group."""
    _check(load().gs_adam_step(n, groups, len(groups), ctypes.byref(hp), int(t), _ptr(last_step), _ptr(active),
                               int(n_active), _stream(stream)), "gs_adam_step")


def gs_adam_step_seen(n, groups, hp: gs_adam_params, t, last_step, seen, stream=None):
    """Deferred step over the Gaussians whose seen flag (device uint8 [n]) is set."""
    _check(load().gs_adam_step_seen(n, groups, len(groups), ctypes.byref(hp), int(t), _ptr(last_step), _ptr(seen),
                                    _stream(stream)), "gs_adam_step_seen")


def gs_adam_flush(n, groups, hp: gs_adam_params, t, last_step, stream=None):
    _check(load().gs_adam_flush(n, groups, len(groups), ctypes.byref(hp), int(t), _ptr(last_step), _stream(stream)),
           "gs_adam_flush")
