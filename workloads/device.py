"""Device placement of seeded inputs (torch is used only for memory)."""
from __future__ import annotations

import numpy as np

from . import Case


def to_dev(a: np.ndarray, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload_experts(case: Case, device="cuda:0"):
    """Generate the expert weights expert by expert straight into device tensors
    ([E,2I,H/2], [E,2I,H/32], [E,H,I/2], [E,H,I/32] uint8)."""
    import torch
    s = case.shape
    E, H, I = s.experts, s.hidden, s.inter
    w13c = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=device)
    w13s = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=device)
    w2c = torch.empty((E, H, I // 2), dtype=torch.uint8, device=device)
    w2s = torch.empty((E, H, I // 32), dtype=torch.uint8, device=device)
    for e in range(E):
        a, b, c, x = case.expert(e)
        w13c[e].copy_(torch.from_numpy(np.array(a)))
        w13s[e].copy_(torch.from_numpy(b))
        w2c[e].copy_(torch.from_numpy(np.array(c)))
        w2s[e].copy_(torch.from_numpy(x))
    return w13c, w13s, w2c, w2s
