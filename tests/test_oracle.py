"""Pins of the CPU oracle to things other than itself (CPU only).

* brute force: dense attention over the un-paged K/V (einsum with an explicit
  mask matrix) and torch's scaled_dot_product_attention in float64;
* closed forms: a single key returns its V row and its score, a constant score
  returns mean(V) and ln(n), a dominant key returns its V row exactly;
* invariants: softmax weights sum to 1, merging split partials reproduces the
  unsplit result for any split count, a physical page permutation leaves the
  result bitwise unchanged;
* the split rule against the trip counts printed in aiter PR #4758's Test
  Result tables, and against a brute-force search (also the shared-prefix
  split rule, whose partials must merge to the unsplit result);
* planted mistakes (wrong slot, dropped scale, top-left causal alignment,
  wrong GQA head map, interleaved KV-head rule, V read from K, flipped merge
  sign, log base 2) each fail one of the pins above.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.reference as ref
from workloads import Workload, bf16_bits_from_f32, generate
from workloads.gen import Inputs, designate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_table(name):
    rows, ctx = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln.strip() for ln in f if ln.strip()]
    header = None
    for ln in lines:
        if ln.startswith("#"):
            if ln.startswith("# context"):
                ctx = int(ln.split()[-1])
            continue
        if header is None:
            header = ln.split()
            continue
        rows.append(dict(zip(header, (int(x) for x in ln.split()))))
    return ctx, rows


# --------------------------------------------------------------------------
# tiny dense problems scattered into a paged pool (test-side construction)
# --------------------------------------------------------------------------

def _wl(B=2, q_len=1, Hq=4, Hkv=2, Dk=16, Dv=16, P=4, ctx=(13, 9), causal=False,
        kv="f32", alias=False, pool=None):
    need = sum(-(-c // P) for c in ctx)
    return Workload(name="tiny", batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim_qk=Dk, head_dim_v=Dv, page_size=P, kv_dtype=kv,
                    context_lens=tuple(ctx), pool_pages=pool or (need + 5),
                    v_aliases_k=alias, causal=causal, seed=7)


def dense_problem(w: Workload, seed=0):
    """Dense per-request K/V (float64 values exactly representable in the
    workload's dtype), scattered into a randomly permuted page pool."""
    rng = np.random.default_rng(seed)

    def draw(shape):
        v = rng.standard_normal(shape).astype(np.float32)
        if w.kv_dtype == "f32":
            return v, v.astype(np.float64)
        bits = bf16_bits_from_f32(v)
        # decode through torch's bfloat16 type (a library routine, not the oracle's)
        dec = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        return bits, dec

    Lmax = max(w.context_lens)
    q_st, q_d = draw((w.batch, w.q_len, w.num_q_heads, w.head_dim_qk))
    K_st, K_d = draw((w.batch, w.num_kv_heads, Lmax, w.head_dim_qk))
    if w.v_aliases_k:
        V_st, V_d = None, K_d[..., :w.head_dim_v]
    else:
        V_st, V_d = draw((w.batch, w.num_kv_heads, Lmax, w.head_dim_v))
    dt = np.float32 if w.kv_dtype == "f32" else np.uint16
    kpool = np.zeros((w.pool_pages, w.num_kv_heads, w.page_size, w.head_dim_qk), dt)
    vpool = None if w.v_aliases_k else np.zeros(
        (w.pool_pages, w.num_kv_heads, w.page_size, w.head_dim_v), dt)
    perm = rng.permutation(w.pool_pages).astype(np.int32)
    pt = np.zeros((w.batch, w.max_pages_per_req), np.int32)
    cur = 0
    for b, L in enumerate(w.context_lens):
        n = -(-L // w.page_size)
        pt[b, :n] = perm[cur:cur + n]
        cur += n
        for t in range(L):
            kpool[pt[b, t // w.page_size], :, t % w.page_size] = K_st[b, :, t]
            if vpool is not None:
                vpool[pt[b, t // w.page_size], :, t % w.page_size] = V_st[b, :, t]
    inp = Inputs(w=w, q=q_st, k_cache=kpool, v_cache=vpool, page_table=pt,
                 context_lens=np.asarray(w.context_lens, np.int32),
                 scale=np.float32(1.0 / math.sqrt(w.head_dim_qk)))
    return inp, q_d, K_d, V_d


def dense_einsum(w, q, K, V, scale):
    """Dense attention with an explicit bottom-right causal mask matrix."""
    g = w.num_q_heads // w.num_kv_heads
    out = np.zeros((w.batch, w.q_len, w.num_q_heads, w.head_dim_v))
    lse = np.zeros((w.batch, w.q_len, w.num_q_heads))
    for b, L in enumerate(w.context_lens):
        Kx = np.repeat(K[b, :, :L], g, axis=0)      # [Hq, L, Dk]
        Vx = np.repeat(V[b, :, :L], g, axis=0)
        s = np.einsum("jhd,htd->jht", q[b], Kx) * scale
        j = np.arange(w.q_len)[:, None]
        t = np.arange(L)[None, :]
        mask = (t <= L - w.q_len + j) if w.causal else np.ones((w.q_len, L), bool)
        s = np.where(mask[:, None, :], s, -np.inf)
        mx = s.max(axis=-1, keepdims=True)
        e = np.exp(s - mx)
        den = e.sum(axis=-1, keepdims=True)
        out[b] = np.einsum("jht,htd->jhd", e / den, Vx)
        lse[b] = (mx + np.log(den))[..., 0]
    return out, lse


def dense_sdpa(w, q, K, V, scale):
    """torch.nn.functional.scaled_dot_product_attention, float64 on the CPU."""
    g = w.num_q_heads // w.num_kv_heads
    out = np.zeros((w.batch, w.q_len, w.num_q_heads, w.head_dim_v))
    for b, L in enumerate(w.context_lens):
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)[None]                    # [1, Hq, ql, Dk]
        kt = torch.from_numpy(np.repeat(K[b, :, :L], g, axis=0))[None]
        vt = torch.from_numpy(np.repeat(V[b, :, :L], g, axis=0).copy())[None]
        j = torch.arange(w.q_len)[:, None]
        t = torch.arange(L)[None, :]
        mask = (t <= L - w.q_len + j) if w.causal else torch.ones(w.q_len, L, dtype=torch.bool)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        out[b] = o[0].permute(1, 0, 2).numpy()
    return out


CASES = [
    dict(),
    dict(kv="bf16"),
    dict(B=3, Hq=8, Hkv=2, Dk=32, Dv=32, P=1, ctx=(1, 7, 20)),
    dict(B=2, q_len=4, Hq=4, Hkv=2, P=4, ctx=(4, 11), causal=True),
    dict(B=2, q_len=3, Hq=6, Hkv=3, P=2, ctx=(5, 16), causal=True, kv="bf16"),
    dict(B=2, Hq=4, Hkv=1, Dk=24, Dv=16, P=1, ctx=(9, 17), alias=True, kv="bf16"),
    dict(B=1, q_len=2, Hq=4, Hkv=4, Dk=8, Dv=12, P=3, ctx=(10,), causal=False),
]


def bruteforce_error(case, oracle_mod=ref):
    w = _wl(**case)
    inp, q, K, V = dense_problem(w)
    scale = float(np.float64(inp.scale))
    o_ref, l_ref = dense_einsum(w, q, K, V, scale)
    o, l = oracle_mod.decode_reference(inp)
    err = max(np.max(np.abs(o - o_ref)), np.max(np.abs(l - l_ref)))
    o_t = dense_sdpa(w, q, K, V, scale)
    return max(err, np.max(np.abs(o - o_t)))


@pytest.mark.parametrize("case", CASES)
def test_bruteforce_dense(case):
    assert bruteforce_error(case) <= 1e-12


def test_weights_sum_to_one():
    rng = np.random.default_rng(3)
    for n in (1, 2, 7, 1000):
        s = rng.standard_normal(n) * 10
        wts, lse = oracle.softmax_weights(s)
        assert abs(wts.sum() - 1.0) <= 1e-12
        assert abs(lse - np.log(np.sum(np.exp(s)))) <= 1e-9 * max(1, abs(lse))


def test_single_key_closed_form():
    for kv in ("f32", "bf16"):
        w = _wl(B=1, ctx=(1,), kv=kv)
        inp, q, K, V = dense_problem(w, seed=4)
        o, l = oracle.decode_reference(inp)
        g = w.num_q_heads // w.num_kv_heads
        for h in range(w.num_q_heads):
            np.testing.assert_array_equal(o[0, 0, h], V[0, h // g, 0])
            s0 = float(np.dot(q[0, 0, h], K[0, h // g, 0])) * float(np.float64(inp.scale))
            assert abs(l[0, 0, h] - s0) <= 1e-13


def test_constant_score_closed_form():
    w = _wl(B=2, ctx=(13, 9), q_len=2, causal=True)
    inp, q, K, V = dense_problem(w, seed=5)
    inp = inp.with_(q=np.zeros_like(inp.q))
    o, l = oracle.decode_reference(inp)
    g = w.num_q_heads // w.num_kv_heads
    for b, L in enumerate(w.context_lens):
        for j in range(w.q_len):
            n = L - w.q_len + 1 + j
            for h in range(w.num_q_heads):
                np.testing.assert_allclose(o[b, j, h], V[b, h // g, :n].mean(axis=0), rtol=0, atol=1e-14)
                assert abs(l[b, j, h] - math.log(n)) <= 1e-13


def test_equal_keys_give_mean():
    w = _wl(B=1, ctx=(11,))
    inp, q, K, V = dense_problem(w, seed=6)
    k = inp.k_cache.copy()
    k[...] = k[inp.page_table[0, 0], :, 0][None, :, None, :]
    o, _ = oracle.decode_reference(inp.with_(k_cache=k))
    g = w.num_q_heads // w.num_kv_heads
    for h in range(w.num_q_heads):
        np.testing.assert_allclose(o[0, 0, h], V[0, h // g, :11].mean(axis=0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("alias", [False, True])
def test_dominant_key_closed_form(alias):
    kw = dict(B=2, Hq=4, Hkv=1, Dk=96 if alias else 64, Dv=32 if alias else 64,
              P=1 if alias else 4, ctx=(40, 29), kv="bf16", alias=alias)
    w = _wl(**kw)
    inp, q, K, V = dense_problem(w, seed=8)
    tok = [[[17]], [[0]]]
    d = designate(inp, tok)
    o, l = oracle.decode_reference(d)
    score_dims = w.head_dim_qk - (w.head_dim_v if alias else 0)
    for b in range(2):
        t = tok[b][0][0]
        page = d.page_table[b, t // w.page_size]
        vrow = oracle.to_f64((d.k_cache if alias else d.v_cache)[page, 0, t % w.page_size][:w.head_dim_v],
                             "bf16")
        for h in range(w.num_q_heads):
            np.testing.assert_array_equal(o[b, 0, h], vrow)
            assert abs(l[b, 0, h] - score_dims) <= 1e-12


@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[4], CASES[5]])
def test_split_merge_reproduces_unsplit(case):
    w = _wl(**case)
    inp, *_ = dense_problem(w, seed=9)
    o, l = oracle.decode_reference(inp)
    for S in (1, 2, 3, 5, 8):
        for A in (1, 2, 4):
            op, lp = oracle.split_reference(inp, S, A)
            om, lm = oracle.merge_reference(op, lp)
            np.testing.assert_allclose(om, o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lm, l, rtol=0, atol=1e-12)


def test_page_permutation_bitwise_invariant():
    w = _wl(B=2, q_len=2, causal=True, kv="bf16", P=2, ctx=(9, 14))
    inp, *_ = dense_problem(w, seed=10)
    rng = np.random.default_rng(11)
    perm = rng.permutation(w.pool_pages)          # new slot of old page p is perm[p]
    k2 = np.empty_like(inp.k_cache)
    v2 = np.empty_like(inp.v_cache)
    k2[perm] = inp.k_cache
    v2[perm] = inp.v_cache
    pt2 = perm[inp.page_table].astype(np.int32)
    a = oracle.decode_reference(inp)
    b = oracle.decode_reference(inp.with_(k_cache=k2, v_cache=v2, page_table=pt2))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_empty_context_and_empty_splits():
    w = _wl(B=2, ctx=(0, 5), P=4)
    inp, *_ = dense_problem(w, seed=12)
    o, l = oracle.decode_reference(inp)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    op, lp = oracle.split_reference(inp, 4, 4)
    # request 1 has 5 keys in 4-key chunks: splits 0 and 1 hold keys, 2 and 3 are empty
    assert np.all(np.isfinite(lp[1, :, :, :2])) and np.all(np.isneginf(lp[1, :, :, 2:]))
    assert np.all(op[1, :, :, 2:] == 0)


# --------------------------------------------------------------------------
# split rule
# --------------------------------------------------------------------------

def test_split_rule_matches_policy_table():
    ctx, rows = read_table("aiter4758_policy_table.txt")
    for r in rows:
        bounds = oracle.split_bounds(ctx, r["splits"], 64)
        first = bounds[0][1] - bounds[0][0]
        assert first % 64 == 0 and first // 64 == r["trips"], r


def test_split_rule_matches_forced_table():
    ctx, rows = read_table("aiter4758_forced_splits.txt")
    for r in rows:
        assert ctx // r["splits"] == r["tok_per_split"]
        assert -(-r["tok_per_split"] // 64) == r["trips"]
        bounds = oracle.split_bounds(ctx, r["splits"], 64)
        assert (bounds[0][1] - bounds[0][0]) // 64 == r["trips"], r


def test_split_rule_bruteforce():
    for L in range(0, 130):
        for S in range(1, 12):
            for A in (1, 2, 3, 16, 64):
                c = A
                while S * c < L:              # smallest multiple of A with S*c >= L
                    c += A
                bounds = oracle.split_bounds(L, S, A)
                assert len(bounds) == S
                exp = [(min(s * c, L), min((s + 1) * c, L)) for s in range(S)]
                assert bounds == exp, (L, S, A)
                # partition of [0, L)
                covered = [t for b, e in bounds for t in range(b, e)]
                assert covered == list(range(L))


def test_fixed_chunk_split_rule_bruteforce():
    """Fixed split length c for every request: the S splits partition the
    first min(L, S*c) keys in order, each non-empty split but the last of a
    request holds exactly c keys, the request holds ceil(L / c) non-empty
    splits, and every later split is empty (begin = end = the end of the
    keys)."""
    for L in range(0, 200):
        for c in (1, 2, 3, 16, 64, 128):
            for S in sorted({1, 2, 5, max(1, -(-L // c)), max(1, -(-L // c)) + 3}):
                bounds = oracle.split_bounds(L, S, 64, chunk=c)
                assert len(bounds) == S
                covered = [t for b, e in bounds for t in range(b, e)]
                assert covered == list(range(min(L, S * c))), (L, c, S)
                lens = [e - b for b, e in bounds]
                live = [n for n in lens if n > 0]
                assert len(live) == min(S, -(-L // c)), (L, c, S)
                assert all(n == c for n in live[:-1])
                first_empty = len(live)
                assert all(n == 0 for n in lens[first_empty:])
                assert all(b == e == min(L, S * c) for b, e in bounds[first_empty:])


def test_fixed_chunk_split_merge_reproduces_unsplit():
    # per-request split counts in proportion to length (ragged batch, causal
    # drafts): the merged partials equal the unsplit result whenever S * c
    # covers the longest request
    for case in (CASES[3], CASES[4], dict(B=3, Hq=8, Hkv=2, Dk=32, Dv=32, P=1, ctx=(1, 7, 20))):
        w = _wl(**case)
        inp, *_ = dense_problem(w, seed=13)
        o, l = oracle.decode_reference(inp)
        for c in (1, 2, 4, 7):
            S = -(-max(w.context_lens) // c)
            op, lp = oracle.split_reference(inp, S, chunk=c)
            mo, ml = oracle.merge_reference(op, lp)
            assert np.max(np.abs(mo - o)) <= 1e-12 and np.max(np.abs(ml - l)) <= 1e-12, (case, c)
            # a split count that stops short of the longest request loses keys
            if S > 1:
                op2, lp2 = oracle.split_reference(inp, S - 1, chunk=c)
                mo2, _ = oracle.merge_reference(op2, lp2)
                assert np.max(np.abs(mo2 - o)) > 1e-6


def test_prefix_split_rule_bruteforce():
    """Shared-prefix splits: the shared set is the split rule over [0, prefix)
    (found by search, as above), the own set the rule over the L - prefix
    remaining keys, shifted by prefix; together they partition [0, L) in
    order.  With prefix = 0 only the own set remains and equals split_bounds."""
    def rule(n, S, A):
        c = A
        while S * c < n:
            c += A
        return [(min(s * c, n), min((s + 1) * c, n)) for s in range(S)]
    for L in range(0, 90, 3):
        for prefix in sorted({0, 1, L // 3, L // 2, L}):
            if prefix > L:
                continue
            for Ss in (1, 2, 5):
                for So in (1, 3, 4):
                    for A in (1, 16, 64):
                        got = oracle.prefix_split_bounds(L, prefix, Ss, So, A)
                        shared = rule(prefix, Ss, A) if prefix > 0 else []
                        own = [(prefix + b, prefix + e) for b, e in rule(L - prefix, So, A)]
                        assert got == shared + own, (L, prefix, Ss, So, A)
                        covered = [t for b, e in got for t in range(b, e)]
                        assert covered == list(range(L))
        assert oracle.prefix_split_bounds(L, 0, 4, 5) == oracle.split_bounds(L, 5)


def test_prefix_split_merge_reproduces_unsplit():
    # partials over the shared keys and each request's own keys merge to the
    # unsplit result (ragged batch, causal drafts, GQA and aliased V)
    for case in (CASES[3], CASES[4], dict(B=3, Hq=8, Hkv=2, Dk=32, Dv=32, P=1, ctx=(9, 7, 20))):
        w = _wl(**case)
        inp, *_ = dense_problem(w, seed=17)
        o, l = oracle.decode_reference(inp)
        lo = min(w.context_lens) - w.q_len + 1
        for prefix in sorted({0, 1, max(0, lo // 2), max(0, lo)}):
            for Ss, So in ((1, 1), (2, 3), (3, 2)):
                op, lp = oracle.split_reference(inp, (Ss if prefix else 0) + So,
                                                bounds_of=lambda L: oracle.prefix_split_bounds(L, prefix, Ss, So))
                mo, ml = oracle.merge_reference(op, lp)
                assert np.max(np.abs(mo - o)) <= 1e-12 and np.max(np.abs(ml - l)) <= 1e-12, (case, prefix)


def test_visible_keys_rule():
    assert oracle.visible_keys(10, 1, 0, True) == 10
    assert [oracle.visible_keys(10, 4, j, True) for j in range(4)] == [7, 8, 9, 10]
    assert [oracle.visible_keys(10, 4, j, False) for j in range(4)] == [10] * 4
    assert oracle.visible_keys(0, 1, 0, True) == 0


# --------------------------------------------------------------------------
# planted mistakes: each must fail a pin
# --------------------------------------------------------------------------

def _planted(monkeypatch, name, fn):
    monkeypatch.setattr(ref, name, fn)


def test_planted_wrong_slot(monkeypatch):
    orig = ref.gather

    def bad(cache, pt_row, kvh, n, P, kv, dims=None):
        t = np.arange(n)
        rows = cache[pt_row[t // P].astype(np.int64), kvh, (t // P) % P]
        return ref.to_f64(rows if dims is None else rows[:, :dims], kv)
    _planted(monkeypatch, "gather", bad)
    assert bruteforce_error(CASES[0]) > 1e-3
    monkeypatch.setattr(ref, "gather", orig)
    assert bruteforce_error(CASES[0]) <= 1e-12


def test_planted_dropped_scale(monkeypatch):
    orig = ref.attend
    _planted(monkeypatch, "attend", lambda qr, K, V, scale, rg: orig(qr, K, V, 1.0, rg))
    assert bruteforce_error(CASES[0]) > 1e-3


def test_planted_top_left_causal(monkeypatch):
    _planted(monkeypatch, "visible_keys", lambda L, ql, j, c: min(L, j + 1) if c else L)
    assert bruteforce_error(CASES[3]) > 1e-3


def test_planted_gqa_head_map(monkeypatch):
    def bad_rows(inp, b, kvh):
        w = inp.w
        idx = [(j, h) for j in range(w.q_len) for h in range(w.num_q_heads) if h % w.num_kv_heads == kvh]
        return idx, np.stack([ref.to_f64(inp.q[b, j, h], w.kv_dtype) for (j, h) in idx])
    _planted(monkeypatch, "_request_rows", bad_rows)
    assert bruteforce_error(CASES[0]) > 1e-3


def test_planted_kv_head_of(monkeypatch):
    # interleaved instead of consecutive groups: query head h on KV head h % H_kv
    _planted(monkeypatch, "kv_head_of", lambda h, hq, hkv: h % hkv)
    assert bruteforce_error(CASES[0]) > 1e-3
    # a single KV head, or one query head per KV head, cannot tell the maps apart
    assert bruteforce_error(CASES[5]) <= 1e-12


def test_planted_v_from_k(monkeypatch):
    def bad_kv(inp, b, kvh, n):
        w = inp.w
        K = ref.gather(inp.k_cache, inp.page_table[b], kvh, n, w.page_size, w.kv_dtype)
        return K, K[:, :w.head_dim_v]
    _planted(monkeypatch, "_kv", bad_kv)
    assert bruteforce_error(CASES[0]) > 1e-3


def test_planted_unshifted_own_splits(monkeypatch):
    # own splits left at [0, L - prefix): keys overlap the shared set and the
    # last prefix keys are never read
    def bad(L, prefix, Ss, So, A=oracle.SPLIT_ALIGN):
        shared = oracle.split_bounds(prefix, Ss, A) if prefix > 0 else []
        return shared + oracle.split_bounds(L - prefix, So, A)
    monkeypatch.setattr(oracle, "prefix_split_bounds", bad)
    with pytest.raises(AssertionError):
        test_prefix_split_rule_bruteforce()
    with pytest.raises(AssertionError):
        test_prefix_split_merge_reproduces_unsplit()


def test_planted_merge_sign():
    w = _wl(**CASES[0])
    inp, *_ = dense_problem(w, seed=9)
    o, _ = oracle.decode_reference(inp)
    op, lp = oracle.split_reference(inp, 3, 2)
    M = lp.max(axis=-1, keepdims=True)
    wts = np.exp(M - lp)                       # flipped sign
    bad = (wts[..., None] * op).sum(-2) / wts.sum(-1)[..., None]
    assert np.max(np.abs(bad - o)) > 1e-3


def test_planted_log2_lse(monkeypatch):
    def bad_weights(s):
        m = np.max(s)
        e = np.exp(s - m)
        return e / e.sum(), m + math.log2(e.sum())
    _planted(monkeypatch, "softmax_weights", bad_weights)
    w = _wl(B=1, ctx=(13,))
    inp, *_ = dense_problem(w, seed=5)
    _, l = ref.decode_reference(inp.with_(q=np.zeros_like(inp.q)))
    assert abs(l[0, 0, 0] - math.log(13)) > 1e-3


# --------------------------------------------------------------------------
# generator sanity (shapes the pages' workloads have)
# --------------------------------------------------------------------------

def test_generated_shapes_small():
    from workloads import get, scaled
    inp = generate(get("gqa_tiny_f32"))
    assert inp.k_cache.shape == (16, 1, 16, 64) and inp.q.dtype == np.float32
    assert sorted(inp.page_table[0].tolist()) == list(range(16))
    w = scaled("mla_b48", batch=16, context_lens=(300,) * 16, prefix_len=200)
    inp = generate(w)
    assert inp.v_cache is None
    # requests of one group share the prefix pages, not the private ones
    assert np.array_equal(inp.page_table[0, :200], inp.page_table[7, :200])
    assert not np.array_equal(inp.page_table[0, :200], inp.page_table[8, :200])
    assert len(set(inp.page_table[0, 200:300]) & set(inp.page_table[1, 200:300])) == 0
