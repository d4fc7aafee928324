"""Upload generated inputs to a torch device (raw bits, no conversion of values)."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .generate import Inputs


@dataclass
class DeviceInputs:
    spec: object
    q_idx: object          # float32 | bfloat16
    w: object              # float32
    k_pool: object         # float32 | bfloat16 | uint8 (fp8 codes)
    k_scale: Optional[object]
    q_sfa: Optional[object]
    kv_pool: Optional[object]
    block_table: Optional[object]   # int32
    q_seq: object          # int32
    q_visible: object      # int32
    block_size: int
    seq_stride: int
    pool_rows: int
    max_visible: int


def tensor_of(arr: np.ndarray, device):
    """numpy array of stored bits -> torch tensor on device (uint16 -> bfloat16 view)."""
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def bits_of(t) -> np.ndarray:
    """torch tensor -> numpy array of its stored bits (bfloat16 -> uint16)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def to_device(inp: Inputs, device="cuda") -> DeviceInputs:
    return DeviceInputs(
        spec=inp.spec, q_idx=tensor_of(inp.q_idx, device), w=tensor_of(inp.w, device),
        k_pool=tensor_of(inp.k_pool, device), k_scale=tensor_of(inp.k_scale, device),
        q_sfa=tensor_of(inp.q_sfa, device), kv_pool=tensor_of(inp.kv_pool, device),
        block_table=tensor_of(inp.block_table, device), q_seq=tensor_of(inp.q_seq, device),
        q_visible=tensor_of(inp.q_visible, device), block_size=inp.spec.block_size,
        seq_stride=inp.seq_stride, pool_rows=int(inp.k_pool.shape[0]),
        max_visible=int(inp.q_visible.max()))
