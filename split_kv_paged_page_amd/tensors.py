"""Fill an attn_decode_desc from torch tensors (shapes and strides only)."""

from __future__ import annotations

from ._lib import ATTN_BF16, ATTN_F32, make_desc


def desc_from_tensors(q, k_cache, v_cache, page_table, *, causal: bool = False):
    """q [B, q_len, H_q, Dk]; k_cache [pages, H_kv, P, Dk]; v_cache
    [pages, H_kv, P, Dv] or None when V is K[..., :Dv] (then the head dim of V
    must be given through ``v_cache`` being None and q's last dim, see
    ``head_dim_v`` below); page_table int32 [B, max_pages]."""
    import torch
    B, q_len, Hq, Dk = q.shape
    pages, Hkv, P, Dk2 = k_cache.shape
    if Dk2 != Dk:
        raise ValueError("q and k_cache head dims differ")
    dt = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}.get(q.dtype)
    if dt is None or k_cache.dtype != q.dtype:
        raise ValueError("q and the KV cache must both be float32 or both bfloat16")
    if k_cache.stride(3) != 1:
        raise ValueError("the head dim of k_cache must be contiguous")
    ks = (k_cache.stride(0), k_cache.stride(1), k_cache.stride(2))
    return dict(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=Dk,
                page_size=P, max_pages_per_req=page_table.shape[1], dtype=dt, causal=causal,
                num_pages=pages, k_strides=ks)


def make_desc_from_tensors(q, k_cache, v_cache, page_table, *, head_dim_v=None, causal=False):
    base = desc_from_tensors(q, k_cache, v_cache, page_table, causal=causal)
    if v_cache is None:
        if head_dim_v is None:
            raise ValueError("head_dim_v is required when V aliases K")
        return make_desc(**base, head_dim_v=head_dim_v, v_aliases_k=True, v_strides=base["k_strides"])
    if v_cache.stride(3) != 1 or v_cache.shape[:3] != k_cache.shape[:3]:
        raise ValueError("v_cache must be [pages, H_kv, P, Dv] with a contiguous head dim")
    vs = (v_cache.stride(0), v_cache.stride(1), v_cache.stride(2))
    return make_desc(**base, head_dim_v=v_cache.shape[3], v_aliases_k=False, v_strides=vs)
