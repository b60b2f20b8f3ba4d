"""Move seeded workloads to the GPU and allocate outputs (torch for memory only)."""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

D = 128


@dataclass
class DeviceLayer:
    S0: "object"      # torch.Tensor [B,H,128,128] f32 (committed state; commit updates it)
    Q: "object"
    K: "object"
    V: "object"
    alpha: "object"
    beta: "object"


@dataclass
class DeviceOutputs:
    O: "object"
    U: "object"
    gamma: "object"


def upload_layer(layer, dtype: str, device="cuda"):
    import torch
    qdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def t(x, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(dt).contiguous()

    return DeviceLayer(S0=t(layer.S0), Q=t(layer.q, qdt), K=t(layer.k, qdt), V=t(layer.v, qdt),
                       alpha=t(layer.alpha), beta=t(layer.beta))


def upload_tree(problem, device="cuda"):
    import torch
    parent = torch.from_numpy(np.ascontiguousarray(problem.parent, dtype=np.int32)).to(device)
    accepted = torch.from_numpy(np.ascontiguousarray(problem.accepted, dtype=np.int32)).to(device)
    return parent, accepted


def alloc_outputs(B: int, H: int, N: int, device="cuda", fill: Optional[float] = None):
    import torch
    mk = (lambda s: torch.full(s, fill, dtype=torch.float32, device=device)) if fill is not None \
        else (lambda s: torch.empty(s, dtype=torch.float32, device=device))
    return DeviceOutputs(O=mk((B, N, H, D)), U=mk((B, N, H, D)), gamma=mk((B, N, H)))


@dataclass
class DeferredLog:
    """The log of the deferred commit and its two header buffers (read one, write the other;
    ``flip()`` after every call).  A fresh log: length 0, scale 1."""
    U: "object"        # [B, H, Lmax, 128] f32
    K: "object"        # [B, H, Lmax, 128] bf16
    scale: list        # two [B, H] f32
    length: list       # two [B] int32
    cur: int = 0

    def headers(self):
        """(scale_in, scale_out, len_in, len_out) for the next call."""
        i, o = self.cur, 1 - self.cur
        return self.scale[i], self.scale[o], self.length[i], self.length[o]

    def flip(self):
        self.cur = 1 - self.cur


def alloc_log(B: int, H: int, Lmax: int, device="cuda") -> DeferredLog:
    import torch
    U = torch.zeros((B, H, Lmax, D), dtype=torch.float32, device=device)
    K = torch.zeros((B, H, Lmax, D), dtype=torch.bfloat16, device=device)
    scale = [torch.ones((B, H), dtype=torch.float32, device=device) for _ in range(2)]
    length = [torch.zeros((B,), dtype=torch.int32, device=device) for _ in range(2)]
    return DeferredLog(U=U, K=K, scale=scale, length=length)
