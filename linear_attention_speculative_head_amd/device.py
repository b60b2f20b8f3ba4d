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
