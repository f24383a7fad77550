"""Copies generated inputs to the GPU as torch tensors (byte-identical to the host arrays).

Input plumbing only: no arithmetic of the method happens here.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


def tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Host array -> device tensor with the same bytes (uint16 becomes bfloat16, uint8 stays)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


@dataclasses.dataclass
class DeviceDecode:
    B: int
    lengths: np.ndarray
    q_idx: torch.Tensor
    q_scale: torch.Tensor
    w: torch.Tensor
    keys: torch.Tensor
    k_scale: torch.Tensor
    q: torch.Tensor
    kv: torch.Tensor
    row_seq: torch.Tensor     # [B] int32 = b
    row_pos: torch.Tensor     # [B] int32 = L_b - 1
    n_valid: torch.Tensor     # [B] int32 = L_b
    block_table: Optional[torch.Tensor] = None
    page_size: int = 0
    seq_stride: int = 0       # contiguous layout: rows per sequence

    @property
    def paged(self):
        return self.block_table is not None

    @property
    def ld(self) -> int:
        """Longest sequence the caches can hold (the score row length)."""
        if self.paged:
            return int(self.block_table.shape[1]) * self.page_size
        return self.seq_stride


def upload_decode(inp, device="cuda") -> DeviceDecode:
    B = inp.B
    L = np.asarray(inp.lengths, dtype=np.int64)
    return DeviceDecode(
        B=B, lengths=L,
        q_idx=tensor(inp.q_idx, device), q_scale=tensor(inp.q_scale, device), w=tensor(inp.w, device),
        keys=tensor(inp.keys, device), k_scale=tensor(inp.k_scale, device),
        q=tensor(inp.q, device), kv=tensor(inp.kv, device),
        row_seq=torch.arange(B, dtype=torch.int32).to(device),
        row_pos=torch.from_numpy((L - 1).astype(np.int32)).to(device),
        n_valid=torch.from_numpy(L.astype(np.int32)).to(device),
        block_table=None if inp.block_table is None else tensor(inp.block_table, device),
        page_size=int(inp.page_size),
        seq_stride=0 if inp.block_table is not None else int(inp.keys.shape[1]),
    )


@dataclasses.dataclass
class DevicePrefill:
    T: int
    q_idx: torch.Tensor
    q_scale: torch.Tensor
    w: torch.Tensor
    keys: torch.Tensor
    k_scale: torch.Tensor
    q: torch.Tensor
    kv: torch.Tensor
    row_seq: torch.Tensor     # [T] int32 = 0
    row_pos: torch.Tensor     # [T] int32 = t
    n_valid: torch.Tensor     # [T] int32 = t + 1
    fp32: bool


def upload_prefill(inp, device="cuda") -> DevicePrefill:
    T = inp.T
    return DevicePrefill(
        T=T, q_idx=tensor(inp.q_idx, device), q_scale=tensor(inp.q_scale, device),
        w=tensor(inp.w, device), keys=tensor(inp.keys, device), k_scale=tensor(inp.k_scale, device),
        q=tensor(inp.q, device), kv=tensor(inp.kv, device),
        row_seq=torch.zeros(T, dtype=torch.int32, device=device),
        row_pos=torch.arange(T, dtype=torch.int32, device=device),
        n_valid=torch.arange(1, T + 1, dtype=torch.int32, device=device),
        fp32=inp.dtype == "f32",
    )
