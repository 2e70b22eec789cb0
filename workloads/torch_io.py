"""Copy generated inputs to torch tensors (host or device); no arithmetic."""

from __future__ import annotations

import numpy as np


def as_tensor(arr: np.ndarray, kv_dtype: str, device):
    import torch
    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def upload(inp, device="cuda") -> dict:
    w = inp.w
    return dict(
        q=as_tensor(inp.q, w.kv_dtype, device),
        k_cache=as_tensor(inp.k_cache, w.kv_dtype, device),
        v_cache=None if inp.v_cache is None else as_tensor(inp.v_cache, w.kv_dtype, device),
        page_table=as_tensor(inp.page_table, "i32", device),
        context_lens=as_tensor(inp.context_lens, "i32", device),
    )
