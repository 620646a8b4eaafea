"""Device buffers for one scene and the calls of one training iteration through the C ABI.

A ``Renderer`` uploads a scene's parameters, allocates every output and workspace buffer once
(torch tensors on the current HIP device), and issues project -> bin (-> cap) -> forward ->
loss gradient -> backward, or project -> bin (-> cap) -> fused, on torch's current stream.
Nothing here computes any part of the method; it only owns memory and marshals arguments.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import gsmi


def ptr(t):
    """Device address of a tensor, or None (a NULL pointer) for an absent optional array."""
    return t.data_ptr() if t is not None else None


class Renderer:
    def __init__(self, scene, settings, device: str = "cuda", instance_capacity: int | None = None,
                 headroom: float = 1.25, early_counts: bool = True, lean: bool = False):
        """lean: request only the optional per-field projection arrays that a later call reads
        (conic/opacity for the cap's scores when the tiles are capped: read from the packed records
        instead it would cost the cap more than the store costs the projection); the packed
        records hold the same values, and projected_host reads the others from there."""
        self.scene = scene
        self.settings = settings
        self.device = torch.device(device)
        self.V = len(scene.cameras)
        cam0 = scene.cameras[0]
        self.W, self.H = cam0.width, cam0.height
        self.tiles_x, self.tiles_y = cam0.tiles_x, cam0.tiles_y
        self.tpv = self.tiles_x * self.tiles_y
        self.n = scene.n
        self.headroom = headroom
        dev = self.device

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

        self.means, self.log_scales, self.quats = up(scene.means), up(scene.log_scales), up(scene.quats)
        self.logits, self.sh = up(scene.opacity_logits), up(scene.sh)
        self.g = gsmi.gs_gaussians(self.n, self.means.data_ptr(), self.log_scales.data_ptr(), self.quats.data_ptr(),
                                   self.logits.data_ptr(), self.sh.data_ptr())
        self.cams = gsmi.make_cameras(scene.cameras)
        self.params = gsmi.make_params(settings)
        V, cap = self.V, max(1, self.n)
        self.capacity = cap
        i32, f32 = torch.int32, torch.float32
        self.vis_count = torch.zeros(V, dtype=i32, device=dev)
        self.inst_count = torch.zeros(V, dtype=torch.int64, device=dev)
        self.vis_ids = torch.empty(V * cap, dtype=i32, device=dev)
        self.lean = lean
        opt = lambda want, k: torch.empty(V * cap * k, dtype=f32, device=dev) if want else None
        self.mean2d = opt(not lean, 2)
        self.conic_opacity = opt(not lean or settings.tile_cap > 0, 4)
        self.color = opt(not lean, 3)
        self.depth = torch.empty(V * cap, dtype=f32, device=dev)
        self.tile_rect = torch.empty(V * cap * 4, dtype=torch.int16, device=dev)
        self.n_tiles = torch.empty(V * cap, dtype=i32, device=dev)
        self.inst_base = torch.empty(V * cap, dtype=i32, device=dev)
        self.raster_rec = torch.empty(V * cap * 16, dtype=f32, device=dev)  # torch allocations are 256-B aligned
        self.proj = gsmi.gs_projected(cap, self.vis_count.data_ptr(), self.inst_count.data_ptr(),
                                      self.vis_ids.data_ptr(), ptr(self.mean2d), ptr(self.conic_opacity),
                                      ptr(self.color), self.depth.data_ptr(), self.tile_rect.data_ptr(),
                                      self.n_tiles.data_ptr(), self.inst_base.data_ptr(), self.raster_rec.data_ptr(),
                                      None)
        # pinned count buffer: the projection copies the counts out before its writing pass
        self.readback = gsmi.gs_readback_create() if early_counts else None
        self.proj.readback = self.readback
        self.ws_proj = torch.empty(gsmi.gs_project_workspace_size(self.n, V), dtype=torch.uint8, device=dev)
        self.ranges = torch.zeros(V * self.tpv * 2, dtype=i32, device=dev)
        self.ranges_capped = torch.zeros(V * self.tpv * 2, dtype=i32, device=dev)
        self.num_capped = torch.zeros(1, dtype=i32, device=dev)
        self.tile_order = torch.zeros(V * self.tpv, dtype=i32, device=dev)
        self.inst_capacity = -1
        self._alloc_bins(instance_capacity if instance_capacity is not None else 0)
        plane = self.H * self.W
        self.image = torch.empty(V * 3 * plane, dtype=f32, device=dev)
        self.t_final = torch.empty(V * plane, dtype=f32, device=dev)
        self.n_contrib = torch.empty(V * plane, dtype=i32, device=dev)
        self.dl = torch.empty(V * 3 * plane, dtype=f32, device=dev)
        self.d_mean2d = torch.empty(V * cap * 2, dtype=f32, device=dev)
        self.d_conic = torch.empty(V * cap * 3, dtype=f32, device=dev)
        self.d_opacity = torch.empty(V * cap, dtype=f32, device=dev)
        self.d_color = torch.empty(V * cap * 3, dtype=f32, device=dev)
        self.grads = gsmi.gs_grads2d(self.d_mean2d.data_ptr(), self.d_conic.data_ptr(), self.d_opacity.data_ptr(),
                                     self.d_color.data_ptr())
        self.loss_sum = torch.zeros(1, dtype=f32, device=dev)
        self.counters = torch.zeros(4, dtype=torch.int64, device=dev)
        self.target = up(scene.target.reshape(-1)) if scene.target is not None else None
        self.dldc_in = up(scene.dldc.reshape(-1)) if scene.dldc is not None else None
        self.info = None

    def __del__(self):
        rb = getattr(self, "readback", None)
        if rb:
            self.readback = None
            try:
                gsmi.gs_readback_destroy(rb)
            except Exception:  # interpreter shutdown: the library may be gone already
                pass

    def _alloc_bins(self, capacity: int):
        if capacity <= self.inst_capacity:
            return
        dev = self.device
        c = max(1, int(capacity))
        self.tile_keys = torch.empty(c, dtype=torch.int32, device=dev)
        self.vals = torch.empty(c, dtype=torch.int32, device=dev)
        self.vals_capped = torch.empty(c, dtype=torch.int32, device=dev)
        self.bins = gsmi.gs_bins(c, 0, self.tile_keys.data_ptr(), self.vals.data_ptr(), self.ranges.data_ptr(),
                                 self.vals_capped.data_ptr(), self.ranges_capped.data_ptr(), self.num_capped.data_ptr(),
                                 self.tile_order.data_ptr())
        self.ws_raster = torch.empty(gsmi.gs_raster_workspace_size(c), dtype=torch.uint8, device=dev)
        self.ws_bin = torch.empty(gsmi.gs_bin_workspace_size(self.capacity, self.V, self.W, self.H, c),
                                  dtype=torch.uint8, device=dev)
        self.inst_capacity = c

    # -- the calls of one iteration ------------------------------------------------------
    def project(self):
        gsmi.gs_project(self.g, self.cams, self.V, self.params, self.proj, self.ws_proj)

    def bin(self):
        st, info, req = gsmi.gs_bin_tiles(self.cams, self.proj, self.V, self.params, self.bins, self.ws_bin)
        if st == 2:  # capacity: grow once and retry
            self._alloc_bins(int(req * self.headroom) + 1024)
            st, info, req = gsmi.gs_bin_tiles(self.cams, self.proj, self.V, self.params, self.bins, self.ws_bin)
            if st != 0:
                raise gsmi.GsError(st, "gs_bin_tiles", gsmi.load().gs_last_error().decode())
        self.info = info
        return info

    def check_bins(self):
        """GS_CHECK: validate the tile lists on the device; returns (status, {kind: violations})."""
        return gsmi.gs_check_bins(self.cams, self.proj, self.V, self.params, self.bins)

    @property
    def use_capped(self) -> int:
        return 1 if self.settings.tile_cap > 0 else 0

    def forward(self, counters: bool = False):
        if counters:
            self.counters.zero_()
        gsmi.gs_raster_fwd(self.cams, self.proj, self.bins, self.V, self.params, self.use_capped, self.image,
                           self.t_final, self.n_contrib, self.counters if counters else None)

    def loss_grad(self, scale: float = 1.0):
        if self.scene.loss == "l1":
            gsmi.gs_loss_l1_grad(self.V, self.W, self.H, self.image, self.target, scale, self.dl, None)
            return self.dl
        return self.dldc_in

    def backward(self, dl):
        gsmi.gs_raster_bwd(self.cams, self.proj, self.bins, self.V, self.params, self.use_capped, self.image,
                           self.t_final, self.n_contrib, dl, self.grads, self.ws_raster)

    def fused(self, scale: float = 1.0, image: bool = True, loss_sum: bool = False, counters: bool = False):
        if counters:
            self.counters.zero_()
        if loss_sum:
            self.loss_sum.zero_()
        if self.scene.loss == "l1":
            mode, src = gsmi.GS_LOSS_L1, self.target
        else:
            mode, src = gsmi.GS_LOSS_EXTERNAL, self.dldc_in
        gsmi.gs_raster_fused(self.cams, self.proj, self.bins, self.V, self.params, self.use_capped, mode, src,
                             scale, self.image if image else None, self.loss_sum if loss_sum else None, self.grads,
                             self.ws_raster, self.counters if counters else None)

    def project_backward(self, seen_only: bool = False):
        """Chain the per-slot 2D gradients of all views to the parameters (gs_project_bwd); with
        seen_only, gs_project_bwd_seen: rows of Gaussians no view sees are left as they are and
        self.seen flags the others."""
        if not hasattr(self, "g3"):
            dev, f32, n = self.device, torch.float32, max(1, self.n)
            nk = self.sh.shape[0]
            self.d_means3 = torch.empty(3 * n, dtype=f32, device=dev)
            self.d_log_scales3 = torch.empty(3 * n, dtype=f32, device=dev)
            self.d_quats3 = torch.empty(4 * n, dtype=f32, device=dev)
            self.d_logits3 = torch.empty(n, dtype=f32, device=dev)
            self.d_sh3 = torch.empty(nk * n, dtype=f32, device=dev)
            self.g3 = gsmi.gs_grads3d(self.d_means3.data_ptr(), self.d_log_scales3.data_ptr(),
                                      self.d_quats3.data_ptr(), self.d_logits3.data_ptr(), self.d_sh3.data_ptr())
        if seen_only:
            if not hasattr(self, "seen"):
                self.seen = torch.empty(max(1, self.n), dtype=torch.uint8, device=self.device)
            gsmi.gs_project_bwd_seen(self.g, self.cams, self.V, self.params, self.proj, self.grads, self.g3,
                                     self.seen)
            return
        gsmi.gs_project_bwd(self.g, self.cams, self.V, self.params, self.proj, self.grads, self.g3)

    def iteration(self, mode: str = "fused", scale: float = 1.0, image: bool = False, project_bwd: bool = False):
        self.project()
        self.bin()
        if mode == "fused":
            self.fused(scale=scale, image=image)
        else:
            self.forward()
            self.backward(self.loss_grad(scale))
        if project_bwd:
            self.project_backward()

    # -- host copies for checks ----------------------------------------------------------
    def projected_host(self, v: int) -> dict:
        cnt = int(self.vis_count[v].item())
        cap = self.capacity
        sl = slice(v * cap, v * cap + cnt)
        rec = self.raster_rec.view(-1, 16)[sl].cpu().numpy()
        # the per-field arrays where requested, else the same values from the packed records
        field = lambda t, k, lo: t.view(-1, k)[sl].cpu().numpy() if t is not None else rec[:, lo:lo + k].copy()
        return dict(
            vis_count=cnt,
            inst_count=int(self.inst_count[v].item()),
            vis_ids=self.vis_ids[sl].cpu().numpy(),
            mean2d=field(self.mean2d, 2, 0),
            conic_opacity=field(self.conic_opacity, 4, 2),
            color=field(self.color, 3, 6),
            depth=self.depth[sl].cpu().numpy(),
            rect=self.tile_rect.view(-1, 4)[sl].cpu().numpy().astype(np.int32) & 0xFFFF,
            n_tiles=self.n_tiles[sl].cpu().numpy(),
            inst_base=self.inst_base[sl].cpu().numpy(),
            raster_rec=rec,
        )

    def bins_host(self, v: int, capped: bool = False) -> dict:
        info = self.info
        r = (self.ranges_capped if capped else self.ranges).view(-1, 2)[v * self.tpv:(v + 1) * self.tpv].cpu().numpy()
        if capped:
            total = int(self.num_capped.item())
            vals_all = self.vals_capped[:total].cpu().numpy()
            nonempty = r[:, 1] > r[:, 0]
            lo = int(r[nonempty, 0].min()) if nonempty.any() else 0
            hi = int(r[nonempty, 1].max()) if nonempty.any() else 0
        else:
            lo, hi = int(info.view_offset[v]), int(info.view_offset[v + 1])
            vals_all = self.vals[:info.num_instances].cpu().numpy()
        rel = r.copy()
        rel[r[:, 1] > r[:, 0]] -= lo
        out = dict(ranges=rel, vals=vals_all[lo:hi])
        if not capped:
            out["tile_keys"] = (self.tile_keys[lo:hi].cpu().numpy().view(np.uint32) - np.uint32(v * self.tpv))
        return out

    def images_host(self):
        V, H, W = self.V, self.H, self.W
        return (self.image.view(V, 3, H, W).cpu().numpy(), self.t_final.view(V, H, W).cpu().numpy(),
                self.n_contrib.view(V, H, W).cpu().numpy())

    def grads3d_host(self) -> dict:
        n, nk = self.n, self.sh.shape[0]
        return dict(d_means=self.d_means3[:3 * n].view(3, n).cpu().numpy(),
                    d_log_scales=self.d_log_scales3[:3 * n].view(3, n).cpu().numpy(),
                    d_quats=self.d_quats3[:4 * n].view(4, n).cpu().numpy(),
                    d_opacity_logits=self.d_logits3[:n].cpu().numpy(),
                    d_sh=self.d_sh3[:nk * n].view(nk, n).cpu().numpy())

    def grads_host(self, v: int) -> dict:
        cnt = int(self.vis_count[v].item())
        cap = self.capacity
        sl = slice(v * cap, v * cap + cnt)
        return dict(d_mean2d=self.d_mean2d.view(-1, 2)[sl].cpu().numpy(),
                    d_conic=self.d_conic.view(-1, 3)[sl].cpu().numpy(),
                    d_opacity=self.d_opacity[sl].cpu().numpy(),
                    d_color=self.d_color.view(-1, 3)[sl].cpu().numpy())
