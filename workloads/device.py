"""Upload generated workload arrays to torch tensors (device plumbing only)."""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from .configs import MoEConfig


def to_tensor(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    """uint16 arrays are bf16 bit patterns, uint8 arrays e4m3 codes."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.uint8:
        t = torch.from_numpy(a)
    else:
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    return t.to(device)


def layer_kwargs(cfg: MoEConfig, arrays: Dict[str, Optional[np.ndarray]], capacity: int, device="cuda"):
    """Keyword arguments of MoELayer for one workload."""
    keys = ("w_g", "b_g", "w1", "w3", "w2", "s1", "s3", "s2", "b1", "b2",
            "sh_w1", "sh_w3", "sh_w2", "sh_s1", "sh_s3", "sh_s2", "sh_b1", "sh_b2")
    weights = {k: to_tensor(arrays.get(k), device) for k in keys}
    return dict(T=cfg.T, d=cfg.d, d_out=cfg.d_out, E=cfg.E, k=cfg.k, kind=cfg.ffn, d_ff=cfg.d_ff,
                gate=cfg.gate, capacity=capacity, n_shared=cfg.n_shared, alpha=cfg.alpha,
                act_dtype=torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16,
                weights=weights, device=device)
