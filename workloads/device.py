"""Move a workloads.Case to the GPU as torch tensors (copies only, no arithmetic)."""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass
class DeviceCase:
    k: torch.Tensor
    v: torch.Tensor
    q: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]
    tree_mask: Optional[torch.Tensor] = None


def tensor(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    """numpy -> torch on `device`; uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_device(case, device="cuda") -> DeviceCase:
    tm = getattr(case, "tree_mask", None)
    return DeviceCase(k=tensor(case.k_pool, device), v=tensor(case.v_pool, device),
                      q=tensor(case.q, device), block_table=tensor(case.block_table, device),
                      seq_lens=tensor(case.seq_lens, device),
                      k_scale=tensor(case.k_scale, device), v_scale=tensor(case.v_scale, device),
                      tree_mask=None if tm is None else tensor(tm.view(np.int64), device))


def to_numpy_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
