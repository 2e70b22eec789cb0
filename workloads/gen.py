"""Seeded generation of paged-KV decode inputs (raw bits, host memory).

Streams for a workload with seed ``s``: ``numpy.random.default_rng(s)`` draws
the page permutation of the pool, then q; the K pool is drawn in chunks of
2^24 values, chunk c from ``default_rng([s, 1, c])``, and the V pool likewise
from ``default_rng([s, 2, c])`` (V is not drawn when it aliases K).  The
chunks are independent streams, so the pools (up to 3.76 GB) are filled by
several threads with the same bits as one thread.  Values are N(0, 1) drawn
as float32; bf16 workloads round them to bf16 with round-to-nearest-even, and
both the oracle and the GPU read the same bf16 bit patterns.

Layouts (all C-contiguous):

* q            [B, q_len, H_q, Dk]          f32 or bf16 bits (uint16)
* k_cache      [pool_pages, H_kv, P, Dk]    f32 or bf16 bits
* v_cache      [pool_pages, H_kv, P, Dv]    (None when V aliases K[..., :Dv])
* page_table   int32 [B, max_pages_per_req], entries past a request's last
               page hold page 0 (never read)
* context_lens int32 [B]
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

from .configs import Workload

_CHUNK = 1 << 24  # values per generation call, fixed so streams are reproducible


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


@dataclass
class Inputs:
    w: Workload
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray | None
    page_table: np.ndarray
    context_lens: np.ndarray
    scale: np.float32

    def with_(self, **kw) -> "Inputs":
        return replace(self, **kw)


def _normal_values(rng: np.random.Generator, shape, kv_dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    f32 = kv_dtype == "f32"
    out = np.empty(n, dtype=np.float32 if f32 else np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        v = rng.standard_normal(e - s, dtype=np.float32)
        out[s:e] = v if f32 else bf16_bits_from_f32(v)
    return out.reshape(shape)


def _normal_pool(seed: int, stream: int, shape, kv_dtype: str) -> np.ndarray:
    """N(0, 1) values of a KV pool; chunk c of 2^24 values comes from
    default_rng([seed, stream, c]), filled by a thread pool (NumPy's
    generators and ufuncs release the GIL on large arrays)."""
    n = int(np.prod(shape))
    f32 = kv_dtype == "f32"
    out = np.empty(n, dtype=np.float32 if f32 else np.uint16)

    def fill(c):
        s = c * _CHUNK
        e = min(n, s + _CHUNK)
        v = np.random.default_rng([seed, stream, c]).standard_normal(e - s, dtype=np.float32)
        out[s:e] = v if f32 else bf16_bits_from_f32(v)

    chunks = -(-n // _CHUNK)
    if chunks <= 1:
        for c in range(chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1, chunks)) as ex:
            list(ex.map(fill, range(chunks)))
    return out.reshape(shape)


def page_table_for(w: Workload, perm: np.ndarray) -> np.ndarray:
    """Assign pool pages to requests from a permutation of the pool.

    Shared-prefix workloads: request b belongs to group b // prefix_group; each
    group's prefix pages are taken first, then every request's private pages.
    """
    P = w.page_size
    if w.pages_needed() > w.pool_pages:
        raise ValueError(f"{w.name}: pool of {w.pool_pages} pages is smaller than the {w.pages_needed()} needed")
    pt = np.zeros((w.batch, w.max_pages_per_req), dtype=np.int32)
    cur = 0
    prefix_pages = {}
    if w.prefix_group:
        assert w.prefix_len % P == 0
        npp = w.prefix_len // P
        for g in range(-(-w.batch // w.prefix_group)):
            prefix_pages[g] = perm[cur:cur + npp]
            cur += npp
    for b, L in enumerate(w.context_lens):
        need = -(-L // P)
        if w.prefix_group:
            pre = prefix_pages[b // w.prefix_group]
            npp = min(len(pre), need)
            pt[b, :npp] = pre[:npp]
            priv = need - npp
            pt[b, npp:need] = perm[cur:cur + priv]
            cur += priv
        else:
            pt[b, :need] = perm[cur:cur + need]
            cur += need
    assert cur == w.pages_needed()
    return pt


def generate(w: Workload) -> Inputs:
    rng = np.random.default_rng(w.seed)
    perm = rng.permutation(w.pool_pages).astype(np.int32)
    pt = page_table_for(w, perm)
    q = _normal_values(rng, (w.batch, w.q_len, w.num_q_heads, w.head_dim_qk), w.kv_dtype)
    k = _normal_pool(w.seed, 1, (w.pool_pages, w.num_kv_heads, w.page_size, w.head_dim_qk), w.kv_dtype)
    v = None
    if not w.v_aliases_k:
        v = _normal_pool(w.seed, 2, (w.pool_pages, w.num_kv_heads, w.page_size, w.head_dim_v), w.kv_dtype)
    ctx = np.asarray(w.context_lens, dtype=np.int32)
    return Inputs(w=w, q=q, k_cache=k, v_cache=v, page_table=pt, context_lens=ctx,
                  scale=np.float32(w.scale))


def _encode(vals: np.ndarray, kv_dtype: str) -> np.ndarray:
    vals = np.asarray(vals, dtype=np.float32)
    return vals if kv_dtype == "f32" else bf16_bits_from_f32(vals)


def designate(inp: Inputs, tokens) -> Inputs:
    """One-hot construction: for request b and KV head h, key ``tokens[b][h]``
    (an iterable of logical key positions) gets +1 on its score dims, every
    other key -1, and q is +1 on the score dims; scale becomes 1.

    The score dims are all of Dk, except when V aliases K: then only the dims
    past Dv carry the score, so the aliased V rows stay random and distinct.
    With a score gap of 2 * (number of score dims) >= 128 every non-designated
    weight underflows to zero in float32.
    """
    w = inp.w
    P = w.page_size
    lo = w.head_dim_v if w.v_aliases_k else 0
    k = inp.k_cache.copy()
    k[..., lo:] = _encode(-np.ones(1, np.float32), w.kv_dtype)[0]
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            for t in tokens[b][h]:
                page = inp.page_table[b, t // P]
                k[page, h, t % P, lo:] = _encode(np.ones(1, np.float32), w.kv_dtype)[0]
    q = inp.q.copy()
    q[...] = _encode(np.zeros(1, np.float32), w.kv_dtype)[0]
    q[..., lo:] = _encode(np.ones(1, np.float32), w.kv_dtype)[0]
    return inp.with_(q=q, k_cache=k, scale=np.float32(1.0))


def ramp(inp: Inputs, top: float, q_gain: float = 1.0) -> Inputs:
    """Scores that rise along the context: the K row of request b's key t is
    multiplied by 1 + (top - 1) * t / (L_b - 1), and q by ``q_gain``.  The
    running max of a split then moves up many times, by small and large steps.
    When V aliases K the V rows scale with their keys.  Requests must not share
    pages (no prefix groups): a shared row would take the last request's factor.
    """
    w = inp.w
    if w.prefix_group:
        raise ValueError("ramp needs private pages")
    P = w.page_size
    as_f32 = (lambda a: a) if w.kv_dtype == "f32" else \
        (lambda a: (a.astype(np.uint32) << np.uint32(16)).view(np.float32))
    k = inp.k_cache.copy()
    for b in range(w.batch):
        L = int(inp.context_lens[b])
        for t in range(L):
            f = np.float32(1.0 + (top - 1.0) * t / max(L - 1, 1))
            page = inp.page_table[b, t // P]
            k[page, :, t % P, :] = _encode(as_f32(k[page, :, t % P, :]) * f, w.kv_dtype)
    q = _encode(as_f32(inp.q) * np.float32(q_gain), w.kv_dtype) if q_gain != 1.0 else inp.q
    return inp.with_(q=q, k_cache=k)
