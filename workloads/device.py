"""Upload a seeded workload to the GPU as torch tensors (plumbing only).

KV pools keep their storage bytes: fp32 -> float32, fp16 -> float16, bf16
bit patterns -> bfloat16 (same 16 bits), fp8 codes (E4M3, E5M2) -> uint8.  Nothing of the method is computed.
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch

from . import BF16, F8, F8E5, F16, F32, Workload

TORCH_KV = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16, F8: torch.uint8,
            F8E5: torch.uint8}


def kv_tensor(a: np.ndarray, dtype: int, device="cuda") -> torch.Tensor:
    if dtype == BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def kv_numpy(t: torch.Tensor, dtype: int) -> np.ndarray:
    """Back to the storage numpy array (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu()
    if dtype == BF16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def i32(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def upload(wl: Workload, device="cuda") -> SimpleNamespace:
    sh = wl.shape
    return SimpleNamespace(
        k_pool=kv_tensor(wl.k_pool, sh.kv_dtype, device),
        v_pool=kv_tensor(wl.v_pool, sh.kv_dtype, device),
        q=torch.from_numpy(np.ascontiguousarray(wl.q, dtype=np.float32)).to(device),
        block_table=i32(wl.block_table, device),
        seq_lens=i32(wl.seq_lens, device),
        k_per_seq=i32(wl.k_per_seq, device),
        meta=torch.zeros((sh.num_phys_pages, sh.num_kv_heads, 2, sh.head_dim),
                         dtype=TORCH_KV[sh.kv_dtype], device=device),
    )
