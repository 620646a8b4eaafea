"""Sparse exchange of per-view 2D gradient records (gs_grad_encode / gs_grad_decode): buffers and
thin calls around the C ABI.  Every step runs in the HIP library."""
from __future__ import annotations

import torch

from . import gsmi


class GradCodec:
    """Encoder output buffers (worst case: every visible slot kept) and owner arrays
    [V][n_owner][...] in the layout of gs_grads2d, indexed by Gaussian."""

    def __init__(self, V: int, capacity: int, n_owner: int, device="cuda:0"):
        self.V, self.capacity, self.n_owner = V, capacity, n_owner
        self.max_records = V * capacity
        i32, f32 = torch.int32, torch.float32
        self.keys = torch.empty(max(1, self.max_records), dtype=i32, device=device)
        self.records = torch.empty(max(1, self.max_records) * 9, dtype=f32, device=device)
        self.view_offset = torch.zeros(V + 1, dtype=i32, device=device)
        self.ws = torch.empty(max(256, gsmi.gs_grad_encode_workspace_size(capacity, V)), dtype=torch.uint8,
                              device=device)
        self.o_mean2d = torch.zeros(V * n_owner * 2, dtype=f32, device=device)
        self.o_conic = torch.zeros(V * n_owner * 3, dtype=f32, device=device)
        self.o_opacity = torch.zeros(V * n_owner, dtype=f32, device=device)
        self.o_color = torch.zeros(V * n_owner * 3, dtype=f32, device=device)
        self.owner = gsmi.gs_grads2d(self.o_mean2d.data_ptr(), self.o_conic.data_ptr(), self.o_opacity.data_ptr(),
                                     self.o_color.data_ptr())

    def encode(self, vis_count, vis_ids, grads: "gsmi.gs_grads2d"):
        gsmi.gs_grad_encode(self.V, self.capacity, vis_count, vis_ids, grads, self.keys, self.records,
                            self.view_offset, self.ws)

    def decode(self):
        gsmi.gs_grad_decode(self.V, self.n_owner, self.max_records, self.view_offset, self.keys, self.records,
                            self.owner)

    def zero_owner(self):
        for t in (self.o_mean2d, self.o_conic, self.o_opacity, self.o_color):
            t.zero_()

    def encoded_host(self) -> dict:
        off = self.view_offset.cpu().numpy()
        n = int(off[-1])
        return dict(view_offset=off, keys=self.keys[:n].cpu().numpy(),
                    records=self.records[:9 * n].view(n, 9).cpu().numpy())

    def owner_host(self):
        """Owner arrays as one [V][n_owner][9] array (mean2d x, y, conic A, B, C, opacity, colour)."""
        V, n = self.V, self.n_owner
        return torch.cat([self.o_mean2d.view(V, n, 2), self.o_conic.view(V, n, 3), self.o_opacity.view(V, n, 1),
                          self.o_color.view(V, n, 3)], dim=2).cpu().numpy()
