"""CPU float64 oracle for split-KV paged decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it.

What it computes.  The pages describe the method as a two-stage decode over a
paged KV cache: stage 1 splits each request's keys across workgroups, and
every split computes Q.K times the scale, keeps the running max and sum of the
softmax and accumulates P.V; stage 2 merges the splits by log-sum-exp, each
output slice re-deriving the same per-row statistics (aiter PR #4758, "[Gluon]
[MLA] Deeper async-copy pipeline in the bh16 stage-1 decode loop": Motivation;
Technical Details, items 1 and 3).  In exact arithmetic split-then-merge equals
plain scaled-dot-product softmax attention over the gathered keys, so the
oracle writes that definition out directly in float64:

    s_t   = scale * sum_d q[d] * k_t[d]
    out   = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m),   m = max_t s_t
    lse   = m + ln sum_t exp(s_t - m)                       (natural log)

and, for the per-split check, the same formulas restricted to each split's
key range, plus the log-sum-exp merge of such partials.

Readings where the pages are silent:
* a request's query row j (of q_len) sees keys [0, L - q_len + 1 + j) when
  causal (bottom-right alignment; the context length counts the draft
  tokens), all L keys otherwise;
* query head h reads KV head h // (H_q / H_kv);
* key t of request b lives at page_table[b][t // P], slot t % P;
* split s of S covers [s*c, min((s+1)*c, L)) with c = A * ceil(ceil(L/S)/A),
  A = 64 keys (the 64-key block the trip counts in the aiter PR's tables
  imply), or with c a fixed split length shared by every request of a
  batch (a request then holds ceil(L/c) non-empty splits); a split with no
  visible key gives out = 0, lse = -inf;
* an empty row (no visible key) gives out = 0, lse = -inf;
* shared-prefix plans (groups of requests whose first keys are the same
  pages, as in the aiter PR's MLA workload, Test Plan): a row's splits are
  those of its group's shared keys [0, prefix) by the split rule, then those
  of its own keys [prefix, L) by the same rule applied to L - prefix and
  shifted by prefix.
"""

from __future__ import annotations

import math

import numpy as np

SPLIT_ALIGN = 64


# --------------------------------------------------------------------------
# value decoding (the stored bits, widened exactly)
# --------------------------------------------------------------------------

def to_f64(arr: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Stored values widened exactly to float64 (bf16 bits are the top half
    of a float32)."""
    if kv_dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    u = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# index rules
# --------------------------------------------------------------------------

def visible_keys(L: int, q_len: int, j: int, causal: bool) -> int:
    """Keys query row j of a request with L keys may attend to."""
    if not causal:
        return max(L, 0)
    return max(0, L - q_len + 1 + j)


def split_bounds(L: int, S: int, A: int = SPLIT_ALIGN, chunk: int | None = None) -> list:
    """[begin, end) of each of the S splits of a request with L keys.

    Every split but the last holds the same whole number of A-key blocks; the
    trip count per stage-1 program is then ceil(L / S / A) as in the aiter
    PR's Test Result tables.

    With ``chunk`` given, every request of a batch cuts its keys into splits
    of that fixed length instead: split s covers [s*chunk, min((s+1)*chunk,
    L)), so a request holds ceil(L / chunk) non-empty splits, in proportion
    to its length, and the splits past them are empty.  (The pages trade the
    split count against each program's walk length; with mixed lengths a
    fixed walk length per split keeps every program's walk equal.)
    """
    if S < 1 or A < 1:
        raise ValueError("S and A must be positive")
    if chunk is not None:
        if chunk < 1:
            raise ValueError("chunk must be positive")
    else:
        chunk = A * (-(-(-(-L // S)) // A)) if L > 0 else A
    out = []
    for s in range(S):
        b = min(s * chunk, max(L, 0))
        e = min((s + 1) * chunk, max(L, 0))
        out.append((b, e))
    return out


def prefix_split_bounds(L: int, prefix: int, S_shared: int, S_own: int, A: int = SPLIT_ALIGN) -> list:
    """Split ranges of a request with L keys whose first ``prefix`` keys are
    shared with its group: the S_shared splits of [0, prefix) (none when
    prefix is 0), then the S_own splits of [prefix, L), each set by the split
    rule of split_bounds."""
    if prefix < 0 or prefix > max(L, 0):
        raise ValueError("prefix must lie in [0, L]")
    shared = split_bounds(prefix, S_shared, A) if prefix > 0 else []
    own = [(prefix + b, prefix + e) for (b, e) in split_bounds(L - prefix, S_own, A)]
    return shared + own


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head that query head h reads: consecutive query heads share one
    (a GQA group of num_q_heads / num_kv_heads heads)."""
    return h // (num_q_heads // num_kv_heads)


# --------------------------------------------------------------------------
# gather (the paged walk, as plain indexing)
# --------------------------------------------------------------------------

def gather(cache: np.ndarray, pt_row: np.ndarray, kvh: int, n: int, page_size: int,
           kv_dtype: str, dims: int | None = None) -> np.ndarray:
    """Rows of keys 0..n-1 of one KV head of one request, float64 [n, D]."""
    t = np.arange(n, dtype=np.int64)
    pages = pt_row[t // page_size].astype(np.int64)
    slots = t % page_size
    rows = cache[pages, kvh, slots]
    if dims is not None:
        rows = rows[:, :dims]
    return to_f64(rows, kv_dtype)


# --------------------------------------------------------------------------
# softmax attention
# --------------------------------------------------------------------------

def softmax_weights(scores: np.ndarray) -> tuple:
    """Normalised weights and log-sum-exp of one row of scores (float64)."""
    m = np.max(scores)
    e = np.exp(scores - m)
    den = np.sum(e)
    return e / den, m + math.log(den)


def attend(qr: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, ranges) -> tuple:
    """Softmax attention of query rows ``qr`` [R, Dk] over key rows K [n, Dk],
    V [n, Dv]; row i only sees keys ranges[i] = (begin, end).  Returns
    (out [R, Dv], lse [R]); an empty range gives zeros and -inf."""
    R = qr.shape[0]
    out = np.zeros((R, V.shape[1]), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if K.shape[0] == 0:
        return out, lse
    scores = (qr @ K.T) * scale
    for i, (b, e) in enumerate(ranges):
        if e <= b:
            continue
        w, lse[i] = softmax_weights(scores[i, b:e])
        out[i] = w @ V[b:e]
    return out, lse


def _request_rows(inp, b: int, kvh: int):
    """Query rows of request b that read KV head kvh, as (row index list of
    (j, h)), float64 matrix [R, Dk]."""
    w = inp.w
    idx = [(j, h) for j in range(w.q_len) for h in range(w.num_q_heads)
           if kv_head_of(h, w.num_q_heads, w.num_kv_heads) == kvh]
    qr = np.stack([to_f64(inp.q[b, j, h], w.kv_dtype) for (j, h) in idx])
    return idx, qr


def _kv(inp, b: int, kvh: int, n: int):
    w = inp.w
    K = gather(inp.k_cache, inp.page_table[b], kvh, n, w.page_size, w.kv_dtype)
    if w.v_aliases_k:
        V = K[:, :w.head_dim_v]
    else:
        V = gather(inp.v_cache, inp.page_table[b], kvh, n, w.page_size, w.kv_dtype)
    return K, V


def decode_reference(inp, requests=None) -> tuple:
    """Unsplit attention for every (request, query position, query head).

    Returns (out [B, q_len, H_q, Dv], lse [B, q_len, H_q]) in float64; with
    ``requests`` only those requests are computed (other entries stay NaN).
    """
    w = inp.w
    scale = float(np.float64(inp.scale))
    out = np.full((w.batch, w.q_len, w.num_q_heads, w.head_dim_v), np.nan)
    lse = np.full((w.batch, w.q_len, w.num_q_heads), np.nan)
    for b in (range(w.batch) if requests is None else requests):
        L = int(inp.context_lens[b])
        for kvh in range(w.num_kv_heads):
            idx, qr = _request_rows(inp, b, kvh)
            K, V = _kv(inp, b, kvh, L)
            ranges = [(0, visible_keys(L, w.q_len, j, w.causal)) for (j, _) in idx]
            o, l = attend(qr, K, V, scale, ranges)
            for i, (j, h) in enumerate(idx):
                out[b, j, h] = o[i]
                lse[b, j, h] = l[i]
    return out, lse


def split_reference(inp, S: int, A: int = SPLIT_ALIGN, requests=None, chunk: int | None = None,
                    bounds_of=None) -> tuple:
    """Per-split normalised partial outputs and log-sum-exps, splits as in
    split_bounds (``chunk``: fixed split length for every request), or as
    ``bounds_of(L)`` gives them (a list of S ranges, e.g. prefix_split_bounds).

    Returns (o_part [B, q_len, H_q, S, Dv], lse_part [B, q_len, H_q, S]).
    """
    w = inp.w
    scale = float(np.float64(inp.scale))
    o_part = np.full((w.batch, w.q_len, w.num_q_heads, S, w.head_dim_v), np.nan)
    lse_part = np.full((w.batch, w.q_len, w.num_q_heads, S), np.nan)
    for b in (range(w.batch) if requests is None else requests):
        L = int(inp.context_lens[b])
        bounds = split_bounds(L, S, A, chunk) if bounds_of is None else bounds_of(L)
        if len(bounds) != S:
            raise ValueError(f"{len(bounds)} split ranges for S = {S}")
        for kvh in range(w.num_kv_heads):
            idx, qr = _request_rows(inp, b, kvh)
            K, V = _kv(inp, b, kvh, L)
            for s, (sb, se) in enumerate(bounds):
                ranges = []
                for (j, _) in idx:
                    n = visible_keys(L, w.q_len, j, w.causal)
                    ranges.append((sb, min(se, n)))
                o, l = attend(qr, K, V, scale, ranges)
                for i, (j, h) in enumerate(idx):
                    o_part[b, j, h, s] = o[i]
                    lse_part[b, j, h, s] = l[i]
    return o_part, lse_part


def merge_reference(o_part: np.ndarray, lse_part: np.ndarray) -> tuple:
    """Log-sum-exp merge of split partials over the split axis (-2 of o_part,
    -1 of lse_part): out = sum_s w_s o_s / sum_s w_s, w_s = exp(lse_s - M),
    lse = M + ln sum_s w_s.  Rows whose splits are all empty give 0, -inf."""
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    M = np.max(lse_part, axis=-1)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    wts = np.where(np.isfinite(lse_part), np.exp(lse_part - Ms[..., None]), 0.0)
    den = np.sum(wts, axis=-1)
    num = np.sum(wts[..., None] * o_part, axis=-2)
    safe = np.where(finite, den, 1.0)
    out = np.where(finite[..., None], num / safe[..., None], 0.0)
    lse = np.where(finite, Ms + np.log(safe), -np.inf)
    return out, lse
