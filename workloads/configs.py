"""Workload shapes for split-KV paged decode.

Workloads that stand in for the traffic the pages measure:

* ``gqa_tiny_f32``   - tiny fp32 GQA decode (4 query heads over 1 KV head,
  head dim 64, 256 keys in 16 pages of 16, fixed 4 splits).
* ``gqa_64k``        - long-context GQA decode, bf16 KV (16 query heads over
  2 KV heads, head dim 128, 65,536 keys, page size 16, pool of 8,192 pages).
* ``mla_b48``        - MLA decode as in aiter PR #4758 (Test Plan, workload
  paragraph): 48 requests of 68,000 keys, groups of 8 requests share a
  63,240-key prefix, page size 1, 576-wide latent keys whose first 512 dims
  are the values.  16 query heads (one full bh16 tile).
* ``mla_b48_ctl``    - the same shape with no sharing: every request owns
  68,000 private keys, so the pool exceeds 2 GiB (64-bit offsets) and logical
  KV bytes equal unique bytes.
* ``mla_b1``         - one request of the MLA shape (68,000 keys, 16 query
  heads): the batch-1 end of the same PR's concurrency sweep (Motivation,
  batch-1 paragraph: at batch 1 the split count alone must fill the CUs).
* ``mla_wide``       - the bh64-class MLA shape (128 query heads, 64 requests
  of 16,384 private keys).
* ``varlen_drafts``  - varlen GQA with 4 causal draft tokens per request,
  32 query heads over 4 KV heads, head dim 256, page size 16.  The context
  lengths are the varlen sweep of rocm-libraries PR #10102 (Technical
  Details, launcher-cache paragraph).
* ``gqa_64k_b8_shared`` - 8 requests of the 64K GQA shape that share their
  first 61,440 keys (one group; prefix caching on GQA, the GQA counterpart
  of the MLA batch-48 sharing).
* ``gqa_64k_d64``    - the 64K GQA shape at head dim 64, bf16: the head dim
  whose 128-byte K rows rocm-libraries PR #10102 pads in LDS (Motivation
  bank table).
* ``prefill_2048x4_d64`` / ``prefill_varlen_d64`` (and ``_d128``) - causal
  prefill attention, the step before decode, at the two batches the same
  PR's varlen sweep drives (Technical Details, launcher-cache paragraph):
  4 sequences of 2,048 tokens, and 6 of 256-2,048.  Every token of a
  sequence is a query row; the query block has max_s = 2,048 rows per
  sequence and a shorter sequence's tokens are its last rows (the earlier
  rows see no key and return 0 / -inf).  16 query heads over 4 KV heads
  (one of the PR's GQA ratios), page size 16.

The MLA batch-48 pool: six distinct 63,240-key prefixes plus 48 private
4,760-key suffixes need 607,920 distinct slots, more than a 400k-token pool
holds.  The request structure defines the work, so the pool is sized to fit
(655,360 slots) and page ids are a seeded permutation of it.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    page_size: int
    kv_dtype: str                 # "f32" or "bf16"; q and out use the same type
    context_lens: tuple           # keys per request (includes the draft tokens)
    pool_pages: int               # pages in the KV pool
    v_aliases_k: bool = False     # MLA: V is the first head_dim_v dims of K
    causal: bool = False          # bottom-right causal among the q_len rows
    num_splits: int = 0           # 0: the planner's policy picks
    seed: int = 0
    prefix_group: int = 0         # requests per shared-prefix group (0: none)
    prefix_len: int = 0           # shared prefix keys per group

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def rows_per_kv_head(self) -> int:
        return self.group * self.q_len

    @property
    def max_pages_per_req(self) -> int:
        return max(1, max(-(-c // self.page_size) for c in self.context_lens))

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim_qk)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.kv_dtype == "f32" else 2

    def kv_bytes_per_token_head(self) -> int:
        """Bytes of K (+ V unless aliased) one key of one KV head occupies."""
        d = self.head_dim_qk + (0 if self.v_aliases_k else self.head_dim_v)
        return d * self.elem_bytes

    def logical_kv_bytes(self) -> int:
        """KV bytes the op must read: every visible key of every KV head once
        per request (shared prefixes are counted once per request)."""
        return sum(self.context_lens) * self.num_kv_heads * self.kv_bytes_per_token_head()

    def pages_needed(self) -> int:
        """Pool pages the page tables take: each group's prefix once, then
        every request's pages past it (see gen.page_table_for)."""
        P = self.page_size
        need = [-(-L // P) for L in self.context_lens]
        if not self.prefix_group:
            return sum(need)
        npp = self.prefix_len // P
        groups = -(-self.batch // self.prefix_group)
        return groups * npp + sum(max(0, n - npp) for n in need)

    def unique_kv_bytes(self) -> int:
        if not self.prefix_group:
            return self.logical_kv_bytes()
        groups = -(-self.batch // self.prefix_group)
        dup = (self.batch - groups) * self.prefix_len
        return (sum(self.context_lens) - dup) * self.num_kv_heads * self.kv_bytes_per_token_head()

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["context_lens"] = list(self.context_lens) if len(set(self.context_lens)) > 1 else \
            f"{len(self.context_lens)} x {self.context_lens[0]}"
        return d


def _mk() -> dict:
    c = {}
    c["gqa_tiny_f32"] = Workload(
        name="gqa_tiny_f32", batch=1, q_len=1, num_q_heads=4, num_kv_heads=1,
        head_dim_qk=64, head_dim_v=64, page_size=16, kv_dtype="f32",
        context_lens=(256,), pool_pages=16, num_splits=4, seed=1)
    c["gqa_64k"] = Workload(
        name="gqa_64k", batch=1, q_len=1, num_q_heads=16, num_kv_heads=2,
        head_dim_qk=128, head_dim_v=128, page_size=16, kv_dtype="bf16",
        context_lens=(65536,), pool_pages=8192, seed=2)
    c["mla_b48"] = Workload(
        name="mla_b48", batch=48, q_len=1, num_q_heads=16, num_kv_heads=1,
        head_dim_qk=576, head_dim_v=512, page_size=1, kv_dtype="bf16",
        context_lens=(68000,) * 48, pool_pages=655360, v_aliases_k=True, seed=3,
        prefix_group=8, prefix_len=63240)
    c["mla_b48_ctl"] = Workload(
        name="mla_b48_ctl", batch=48, q_len=1, num_q_heads=16, num_kv_heads=1,
        head_dim_qk=576, head_dim_v=512, page_size=1, kv_dtype="bf16",
        context_lens=(68000,) * 48, pool_pages=48 * 68000, v_aliases_k=True, seed=33)
    c["mla_b1"] = Workload(
        name="mla_b1", batch=1, q_len=1, num_q_heads=16, num_kv_heads=1,
        head_dim_qk=576, head_dim_v=512, page_size=1, kv_dtype="bf16",
        context_lens=(68000,), pool_pages=68000, v_aliases_k=True, seed=42)
    c["mla_wide"] = Workload(
        name="mla_wide", batch=64, q_len=1, num_q_heads=128, num_kv_heads=1,
        head_dim_qk=576, head_dim_v=512, page_size=1, kv_dtype="bf16",
        context_lens=(16384,) * 64, pool_pages=64 * 16384, v_aliases_k=True, seed=4)
    c["varlen_drafts"] = Workload(
        name="varlen_drafts", batch=6, q_len=4, num_q_heads=32, num_kv_heads=4,
        head_dim_qk=256, head_dim_v=256, page_size=16, kv_dtype="bf16",
        context_lens=(256, 512, 768, 1024, 1536, 2048), pool_pages=768, causal=True, seed=5)
    for d in (64, 128):
        c[f"prefill_2048x4_d{d}"] = Workload(
            name=f"prefill_2048x4_d{d}", batch=4, q_len=2048, num_q_heads=16, num_kv_heads=4,
            head_dim_qk=d, head_dim_v=d, page_size=16, kv_dtype="bf16",
            context_lens=(2048,) * 4, pool_pages=1024, causal=True, seed=7)
        c[f"prefill_varlen_d{d}"] = Workload(
            name=f"prefill_varlen_d{d}", batch=6, q_len=2048, num_q_heads=16, num_kv_heads=4,
            head_dim_qk=d, head_dim_v=d, page_size=16, kv_dtype="bf16",
            context_lens=(256, 512, 768, 1024, 1536, 2048), pool_pages=768, causal=True, seed=8)
    c["gqa_64k_b8_shared"] = Workload(
        name="gqa_64k_b8_shared", batch=8, q_len=1, num_q_heads=16, num_kv_heads=2,
        head_dim_qk=128, head_dim_v=128, page_size=16, kv_dtype="bf16",
        context_lens=(65536,) * 8, pool_pages=3840 + 8 * 256, seed=9, prefix_group=8, prefix_len=61440)
    c["gqa_64k_d64"] = Workload(
        name="gqa_64k_d64", batch=1, q_len=1, num_q_heads=16, num_kv_heads=2,
        head_dim_qk=64, head_dim_v=64, page_size=16, kv_dtype="bf16",
        context_lens=(65536,), pool_pages=8192, seed=6)
    return c


CONFIGS = _mk()


def get(name: str) -> Workload:
    return CONFIGS[name]


def scaled(name: str, context_lens=None, pool_pages=None, batch=None, prefix_len=None,
           seed=None, num_splits=None, **kw) -> Workload:
    """The named workload with smaller contexts/pool, same heads, dims and dtype."""
    w = CONFIGS[name]
    upd = dict(kw)
    if batch is not None:
        upd["batch"] = batch
        if context_lens is None:
            context_lens = (w.context_lens[0],) * batch
    if context_lens is not None:
        upd["context_lens"] = tuple(int(x) for x in context_lens)
        upd["batch"] = len(upd["context_lens"])
    if prefix_len is not None:
        upd["prefix_len"] = prefix_len
    if seed is not None:
        upd["seed"] = seed
    if num_splits is not None:
        upd["num_splits"] = num_splits
    w2 = dataclasses.replace(w, name=w.name + "_scaled", **upd)
    if pool_pages is None:
        need = sum(-(-c // w2.page_size) for c in w2.context_lens)
        pool_pages = 2 * need + 3
    return dataclasses.replace(w2, pool_pages=pool_pages)
