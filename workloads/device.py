"""Copies workload arrays to the GPU as torch tensors (plumbing, no arithmetic).

bf16 bit patterns travel as int16 tensors; the library reads their bytes.
"""
import numpy as np
import torch


def to_device(x: np.ndarray, device="cuda"):
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def upload_attn_case(case, device="cuda"):
    """Device tensors of an AttnCase: q1, q2, a, k_cache, v_cache, block_table, ctx_lens."""
    return {name: to_device(getattr(case, name), device)
            for name in ("q1", "q2", "a", "k_cache", "v_cache", "block_table", "ctx_lens")}
