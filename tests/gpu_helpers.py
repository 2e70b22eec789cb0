"""Helpers for the GPU tests: upload seeded inputs, call the C ABI, compare
with the oracle.  Nothing here computes attention."""

from __future__ import annotations

import sys

import numpy as np

import split_kv_paged_page_amd as sk
from workloads.torch_io import upload


def say(msg: str):
    """Name the GPU step about to run (flushed, so it survives a crash)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def validate_inputs(inp):
    """Host-side precondition check before any kernel reads these inputs."""
    w = inp.w
    P = w.page_size
    pool = inp.k_cache.shape[0]
    for b, L in enumerate(inp.context_lens):
        L = int(L)
        assert 0 <= L <= inp.page_table.shape[1] * P, (b, L)
        used = inp.page_table[b, : -(-L // P)]
        assert used.size == 0 or (used.min() >= 0 and used.max() < pool), b


class Decode:
    """One uploaded problem + plan; run() calls attn_decode_run."""

    def __init__(self, inp, num_splits=0, flags=0, max_splits=None, max_context_len=None, relayout=None,
                 lens=False, host_lens=None):
        import torch
        validate_inputs(inp)
        self.inp = inp
        w = inp.w
        self.t = upload(inp, "cuda")
        if relayout is not None:     # other strides for the same cache contents
            self.t = relayout(self.t)
        t = self.t
        self.desc = sk.make_desc_from_tensors(t["q"], t["k_cache"], t["v_cache"], t["page_table"],
                                              head_dim_v=w.head_dim_v, causal=w.causal)
        mx = int(max(inp.context_lens)) if len(inp.context_lens) else 0
        if max_context_len is not None:
            mx = max_context_len
        if lens:     # the batch's lengths known on the host: the policy may fix one split length
            hl = [int(x) for x in (inp.context_lens if host_lens is None else host_lens)]
            self.plan = sk.attn_decode_plan_lens(self.desc, hl, max_splits or num_splits, flags)
        else:
            self.plan = sk.attn_decode_plan(self.desc, mx, max_splits or num_splits, flags)
        self.S = num_splits or self.plan.num_splits
        self.chunk = self.plan.split_chunk or None   # fixed split length, for the oracle's split rule
        self.dtype = torch.float32 if w.kv_dtype == "f32" else torch.bfloat16
        self.ws = torch.empty(self.plan.workspace_bytes // 4, dtype=torch.float32, device="cuda")
        # With the in-kernel merge the workspace starts with its counters,
        # which poisoning leaves alone; they are zeroed once here.
        self.fused = bool(flags & sk.ATTN_PLAN_FUSED_MERGE)
        self.counter_words = sk.attn_decode_workspace_layout(self.plan, self.S)[0] // 4 if self.fused else 0
        if self.fused:
            self.ws[:self.counter_words].fill_(float("nan"))   # the init call must clear them
            sk.attn_decode_workspace_init(self.plan, self.ws)
            torch.cuda.synchronize()
        self.out = torch.empty((w.batch, w.q_len, w.num_q_heads, w.head_dim_v), dtype=self.dtype,
                               device="cuda")
        self.lse = torch.empty((w.batch, w.q_len, w.num_q_heads), dtype=torch.float32, device="cuda")
        self.partials_written = False

    @property
    def v(self):
        return self.t["k_cache"] if self.t["v_cache"] is None else self.t["v_cache"]

    def counters(self) -> np.ndarray:
        """The in-kernel merge's counters (one per request, KV head and head tile)."""
        w = self.inp.w
        n = w.batch * w.num_kv_heads * self.plan.head_tiles
        return self.ws[:n].cpu().numpy().view(np.uint32)

    def poison(self):
        self.ws[self.counter_words:].fill_(float("nan"))
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))

    def run(self, num_splits=None, poison=True):
        import torch
        if poison:
            self.poison()
        t = self.t
        # one split: stage 1 writes the output directly, no partials
        self.partials_written = (num_splits or self.S) > 1
        sk.attn_decode_run(self.plan, t["q"], t["k_cache"], self.v, t["page_table"], t["context_lens"],
                           float(self.inp.scale), num_splits or self.S, self.out, self.lse, self.ws)
        torch.cuda.synchronize()
        return self

    def partials(self, num_splits=None):
        import torch
        t = self.t
        sk.attn_decode_partials(self.plan, t["q"], t["k_cache"], self.v, t["page_table"], t["context_lens"],
                                float(self.inp.scale), num_splits or self.S, self.ws)
        torch.cuda.synchronize()
        self.partials_written = True

    def merge(self, num_splits=None):
        import torch
        sk.attn_decode_merge(self.plan, num_splits or self.S, self.ws, self.out, self.lse)
        torch.cuda.synchronize()

    def out_f64(self):
        import torch
        return self.out.to(torch.float64).cpu().numpy()

    def lse_f64(self):
        return self.lse.double().cpu().numpy()

    def used_ws_bits(self, num_splits=None) -> np.ndarray:
        """Bit patterns of the workspace regions the kernels write (o_part and
        lse_part; the alignment padding between them stays untouched)."""
        S = num_splits or self.S
        w = self.inp.w
        o_off, l_off, _ = sk.attn_decode_workspace_layout(self.plan, S)
        rows = w.batch * w.q_len * w.num_q_heads
        ws = self.ws.cpu().numpy().view(np.int32)
        return np.concatenate([ws[o_off // 4: o_off // 4 + rows * S * w.head_dim_v],
                               ws[l_off // 4: l_off // 4 + rows * S]])

    def split_parts(self, num_splits=None):
        """(o_part [B, q_len, Hq, S, Dv], lse_part [B, q_len, Hq, S]) from the workspace."""
        S = num_splits or self.S
        w = self.inp.w
        o_off, l_off, _ = sk.attn_decode_workspace_layout(self.plan, S)
        rows = w.batch * w.q_len * w.num_q_heads
        ws = self.ws.cpu().numpy()
        o = ws[o_off // 4: o_off // 4 + rows * S * w.head_dim_v].reshape(
            w.batch, w.q_len, w.num_q_heads, S, w.head_dim_v)
        l_ = ws[l_off // 4: l_off // 4 + rows * S].reshape(w.batch, w.q_len, w.num_q_heads, S)
        return o.astype(np.float64), l_.astype(np.float64)


def row_rel_err(y, ref):
    """Max over rows of max_d |y - ref| / max_d |ref| (rows = all but the last axis).
    Rows whose reference is all zero (no visible key) must match exactly."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape
    assert not np.isnan(y).any(), "NaN in output: a value was never written"
    num = np.max(np.abs(y - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    zero = den == 0
    if zero.any():
        assert np.all(num[zero] == 0)
    return float(np.max(np.where(zero, 0.0, num / np.where(zero, 1.0, den))))


def lse_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert not np.isnan(y).any(), "NaN in lse"
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(y), ninf), "empty rows/splits must be -inf on both sides"
    d = np.abs(y[~ninf] - ref[~ninf])
    return float(d.max()) if d.size else 0.0


def tol_for(w) -> float:
    return 1e-5 if w.kv_dtype == "f32" else 1e-2
