"""Adam state over parameter groups (gs_adam_step / gs_adam_flush): moment buffers, the deferred
update's per-Gaussian step counter and thin calls around the C ABI.  Every step runs in the HIP
library."""
from __future__ import annotations

import torch

from . import gsmi


class AdamState:
    """groups: list of (param tensor [rows * n], grad tensor [rows * n], rows, lr) on one device."""

    def __init__(self, n: int, groups, beta1=0.9, beta2=0.999, eps=1e-15, deferred: bool = False):
        self.n = n
        dev = groups[0][0].device
        self.m = [torch.zeros_like(p) for p, _, _, _ in groups]
        self.v = [torch.zeros_like(p) for p, _, _, _ in groups]
        self.groups = (gsmi.gs_adam_group * len(groups))(*[
            gsmi.gs_adam_group(p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(), rows, float(lr))
            for (p, g, rows, lr), m, v in zip(groups, self.m, self.v)])
        self._keep = groups
        self.hp = gsmi.gs_adam_params(beta1, beta2, eps)
        self.last_step = torch.zeros(max(1, n), dtype=torch.int32, device=dev) if deferred else None
        self.t = 0

    def step(self, active=None, seen=None):
        """One step; with a deferred state and `active` (device int32 ids), only those Gaussians, or
        with `seen` (device uint8 [n] flags, as gs_project_bwd_seen writes them), only the flagged
        ones."""
        self.t += 1
        if seen is not None:
            if self.last_step is None:
                raise ValueError("seen flags need a deferred state")
            gsmi.gs_adam_step_seen(self.n, self.groups, self.hp, self.t, self.last_step, seen)
            return
        gsmi.gs_adam_step(self.n, self.groups, self.hp, self.t, self.last_step, active,
                          0 if active is None else active.numel())

    def flush(self):
        if self.last_step is not None and self.t > 0:
            gsmi.gs_adam_flush(self.n, self.groups, self.hp, self.t, self.last_step)
