"""Device copies of one SGMV call's inputs (torch tensors on the GPU) and the calls that
run it through libsgmv.  Accepts any object with the fields of ``workloads.Problem``
(name, dtype, ids, x, y, A, B, scale)."""
from __future__ import annotations

import dataclasses

import numpy as np

from . import sgmv


@dataclasses.dataclass
class DeviceProblem:
    dtype: str
    ids: np.ndarray
    x: object       # torch [n, h_in]
    y0: object      # torch [n, h_out], the input value (kept unmodified)
    A: object       # torch [P, r, h_in]
    B: object       # torch [P, h_out, r]
    scale: float
    batch: sgmv.Batch

    @classmethod
    def upload(cls, p, device="cuda", identity_perm: bool = False, ld_pad: int = 0):
        """Copy a problem to the device.  ``ld_pad`` > 0 stores x and y with row strides
        h + ld_pad (views into wider buffers)."""
        import torch

        def rows(a):
            t = sgmv.as_tensor(a, p.dtype)
            if ld_pad:
                wide = torch.zeros((t.shape[0], t.shape[1] + ld_pad), dtype=t.dtype)
                wide[:, : t.shape[1]] = t
                return wide.to(device)[:, : t.shape[1]]
            return t.to(device)

        x, y0 = rows(p.x), rows(p.y)
        A = sgmv.as_tensor(p.A, p.dtype, device)
        B = sgmv.as_tensor(p.B, p.dtype, device)
        batch = sgmv.Batch.build(p.ids, A, B, identity_perm=identity_perm)
        return cls(p.dtype, p.ids, x, y0, A, B, float(p.scale), batch)

    def fresh_y(self):
        y = self.y0.clone() if self.y0.is_contiguous() else self._clone_strided(self.y0)
        return y

    @staticmethod
    def _clone_strided(t):
        import torch
        wide = torch.empty((t.shape[0], t.stride(0)), dtype=t.dtype, device=t.device)
        out = wide[:, : t.shape[1]]
        out.copy_(t)
        return out

    def lora_add(self, y=None, workspace=None, scale=None):
        y = self.fresh_y() if y is None else y
        sgmv.lora_add(y, self.x, self.batch, self.scale if scale is None else scale, workspace)
        return y

    def lora_add_pool(self, y=None, workspace=None, scale=None, ids=None):
        """The device-id path (one launch for n <= 64, device sort + table kernels up to
        4096 rows)."""
        import torch
        y = self.fresh_y() if y is None else y
        if ids is None:
            ids = torch.as_tensor(self.ids, dtype=torch.int32, device=self.x.device)
        sgmv.lora_add_pool(y, self.x, ids, self.A, self.B,
                           self.scale if scale is None else scale, workspace)
        return y

    def lora_add_host_ids(self, y=None, workspace=None, scale=None, ids=None):
        """The host-id decode path (n <= 64, ids in the launch's kernel arguments)."""
        y = self.fresh_y() if y is None else y
        sgmv.lora_add_host_ids(y, self.x, self.ids if ids is None else ids, self.A, self.B,
                               self.scale if scale is None else scale, workspace)
        return y

    def shrink(self, workspace=None):
        return sgmv.shrink(self.x, self.batch, workspace=workspace)

    def expand(self, v, y=None, scale=None):
        y = self.fresh_y() if y is None else y
        sgmv.expand(y, v, self.batch, self.scale if scale is None else scale)
        return y


def to_numpy_storage(t, dtype: str) -> np.ndarray:
    """A device tensor back in the generator's storage format (float16 / uint16 bits)."""
    import torch
    c = t.detach().contiguous().cpu()
    if dtype == "f16":
        return c.numpy().astype(np.float16, copy=False)
    return c.view(torch.int16).numpy().view(np.uint16)
