"""Copy a seeded workload to GPU memory (torch tensors, same bytes)."""

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .synthetic import Inputs


@dataclass
class DeviceInputs:
    q: torch.Tensor            # float32 or bfloat16 [B][Hq][d]
    k_pool: torch.Tensor       # float32 / bfloat16 / uint8 [N][16][Hkv][d]
    v_pool: torch.Tensor
    k_scale: Optional[torch.Tensor]  # float32 [N][Hkv][16]
    v_scale: Optional[torch.Tensor]
    block_table: torch.Tensor  # int32 [B][max_blocks]
    context_lens: torch.Tensor  # int32 [B]


def _dev(a: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def to_device(inp: Inputs, device="cuda") -> DeviceInputs:
    return DeviceInputs(
        q=_dev(inp.q, device), k_pool=_dev(inp.k_pool, device), v_pool=_dev(inp.v_pool, device),
        k_scale=None if inp.k_scale is None else _dev(inp.k_scale, device),
        v_scale=None if inp.v_scale is None else _dev(inp.v_scale, device),
        block_table=_dev(inp.block_table, device), context_lens=_dev(inp.context_lens, device),
    )
