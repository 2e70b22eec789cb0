"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Tolerances: max over output rows of max|y - y_ref| / max|y_ref| <= 1e-2 for
bf16 inputs (fp32 accumulation, bf16 output) and <= 1e-5 for fp32; final and
per-split log-sum-exp within 1e-3 absolute, -inf exactly where a row or split
has no visible key.  Page gather and split boundaries are checked bit-exactly
with the one-hot construction.  Outputs and workspace are NaN-filled before
every run, so a value the kernels skip cannot pass.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import Decode, lse_err, row_rel_err, say, tol_for
from workloads import generate, get, scaled
from workloads.gen import designate, ramp

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def small_cases():
    return {
        "gqa_tiny_f32": get("gqa_tiny_f32"),
        "gqa_64k_s5000": scaled("gqa_64k", context_lens=(5000,), pool_pages=1024),
        "gqa_64k_b3_ragged": scaled("gqa_64k", context_lens=(1, 777, 4100), pool_pages=1024, seed=21),
        "mla_b48_b16": scaled("mla_b48", batch=16, context_lens=(1000,) * 16, prefix_len=700),
        "mla_wide_b4": scaled("mla_wide", context_lens=(777, 1, 300, 2049)),
        "varlen_drafts": get("varlen_drafts"),
        # bf16 groups that leave part of a 16-row matrix-core tile empty (4, 6,
        # 12 rows; 20 rows: a second tile with 4), at head dims 128, 256 and
        # the MLA 576/512
        "gqa_g4_bf16": scaled("gqa_64k", context_lens=(3000, 1, 777), num_q_heads=8, seed=22),
        "gqa_g6_bf16": scaled("gqa_64k", context_lens=(2500, 130), num_q_heads=12, seed=23),
        "gqa_g12_bf16": scaled("gqa_64k", context_lens=(4100, 65), num_q_heads=24, seed=24),
        "gqa_g20_bf16": scaled("gqa_64k", context_lens=(1500, 2049), num_q_heads=40, seed=25),
        "d256_g8": scaled("varlen_drafts", context_lens=(700, 2049, 64), q_len=1, causal=False, seed=30),
        "mla_h4": scaled("mla_b48", context_lens=(3000, 1, 2100), num_q_heads=4, prefix_len=0, prefix_group=0,
                         seed=29),
        "gqa_d64_bf16": scaled("gqa_64k_d64", context_lens=(4100, 1, 700), seed=32),
        # one request with 16 and 20 rows per KV head: the ring shape where a
        # batch takes key streams
        "mla_h16_b1": scaled("mla_b48", context_lens=(6000,), prefix_len=0, prefix_group=0, seed=40),
        "mla_h16_b4": scaled("mla_b48", context_lens=(3000, 1, 2100, 5000), prefix_len=0, prefix_group=0,
                             seed=43),
        "gqa_g20_b1": scaled("gqa_64k", context_lens=(7000,), num_q_heads=40, seed=41),
        # causal prefill: every token a query row, shorter sequences right-aligned
        "prefill_small_d64": scaled("prefill_varlen_d64", context_lens=(300, 129, 64, 1), q_len=300, seed=34),
        "prefill_small_d128": scaled("prefill_2048x4_d128", context_lens=(257, 257), q_len=257, seed=35),
        # 80 and 120 rows per KV head: a second head tile with 16 and 56 rows
        "prefill_q20_d64": scaled("prefill_varlen_d64", context_lens=(300, 20, 77), q_len=20, seed=36),
        "prefill_q30_d128": scaled("prefill_2048x4_d128", context_lens=(500, 30), q_len=30, seed=37),
        # fp32 runs on the vector ALUs: 8 and 16 rows at head dim 128
        "gqa_f32_g8": scaled("gqa_64k", context_lens=(3000, 1, 777), kv_dtype="f32", seed=28),
        "gqa_f32_g16": scaled("gqa_64k", context_lens=(2100, 300), num_q_heads=32, kv_dtype="f32", seed=31),
        # ragged batches whose plans with known lengths take a fixed split
        # length (320 keys on the matrix cores, 192 on the vector ALUs)
        "gqa_bf16_ragged8": scaled("gqa_64k", context_lens=(9000, 100, 3000, 6000, 1, 12000, 500, 7000), seed=38),
        "gqa_f32_ragged6": scaled("gqa_64k", context_lens=(20000, 1000, 5000, 300, 12000, 7000), kv_dtype="f32",
                                  seed=39),
    }


_INPUTS = {}


def inputs(name, w):
    if name not in _INPUTS:
        _INPUTS[name] = generate(w)
    return _INPUTS[name]


def check_against_oracle(d: Decode, tol, S=None, requests=None, check_splits=True):
    inp = d.inp
    S = S or d.S
    ro, rl = oracle.decode_reference(inp, requests=requests)
    sel = slice(None) if requests is None else list(requests)
    e_out = row_rel_err(d.out_f64()[sel], ro[sel])
    e_lse = lse_err(d.lse_f64()[sel], rl[sel])
    assert e_out <= tol, f"output rel err {e_out:.3e} > {tol}"
    assert e_lse <= 1e-3, f"lse err {e_lse:.3e}"
    if check_splits and d.partials_written:
        po, pl = oracle.split_reference(inp, S, requests=requests, chunk=d.chunk)
        go, gl = d.split_parts(S)
        if d.plan.live_splits > 0:
            # split table: request b writes its first n_b slots only; the
            # oracle's later splits must hold no key (the table covers all)
            for b in (range(inp.w.batch) if requests is None else requests):
                n_b = d.plan.split_start[b + 1] - d.plan.split_start[b]
                assert np.all(np.isneginf(pl[b, ..., n_b:])), b
                go[b, ..., n_b:, :] = po[b, ..., n_b:, :]
                gl[b, ..., n_b:] = pl[b, ..., n_b:]
        gl_ = gl[sel]
        go_ = go[sel]
        e_po = row_rel_err(go_, po[sel])
        e_pl = lse_err(gl_, pl[sel])
        assert e_po <= tol, f"per-split output rel err {e_po:.3e}"
        assert e_pl <= 1e-3, f"per-split lse err {e_pl:.3e}"
        # planted mistake in the oracle: a split rule on 32-key blocks (a split
        # length 64 keys longer, for a plan with a fixed split length) must not
        # agree with the kernel wherever the two rules differ
        lens_sel = inp.context_lens if requests is None else inp.context_lens[list(requests)]
        if S > 1 and d.chunk:
            bo, bl = oracle.split_reference(inp, S, requests=requests, chunk=d.chunk + 64)
            if any(int(L) > d.chunk for L in lens_sel):
                fin = np.isfinite(bl[sel]) & np.isfinite(gl_)
                assert np.max(np.abs(bl[sel][fin] - gl_[fin]), initial=0) > 1e-3 or \
                    np.isneginf(bl[sel]).sum() != np.isneginf(gl_).sum()
        elif S > 1:
            bo, bl = oracle.split_reference(inp, S, A=32, requests=requests)
            differs = any(oracle.split_bounds(int(L), S, 32) != oracle.split_bounds(int(L), S, 64)
                          for L in (inp.context_lens if requests is None else inp.context_lens[list(requests)]))
            if differs:
                fin = np.isfinite(bl[sel]) & np.isfinite(gl_)
                assert np.max(np.abs(bl[sel][fin] - gl_[fin]), initial=0) > 1e-3 or \
                    np.isneginf(bl[sel]).sum() != np.isneginf(gl_).sum()
    return e_out, e_lse


# ragged batches planned with their lengths known on the host: the policy
# gives every request the same split length (per-request split counts)
LENS_CASES = ["gqa_64k_b3_ragged", "mla_wide_b4", "varlen_drafts", "d256_g8", "prefill_small_d64",
              "gqa_bf16_ragged8", "gqa_f32_ragged6"]


@pytest.mark.parametrize("name", LENS_CASES)
def test_parity_small_lens_plans(name):
    w = small_cases()[name]
    inp = inputs(name, w)
    say(f"parity_small lens plan {name} B={w.batch} ctx={w.context_lens[:6]} run")
    d = Decode(inp, lens=True).run()
    e_out, e_lse = check_against_oracle(d, tol_for(w))
    print(f"{name}: S={d.S} chunk={d.plan.split_chunk} out {e_out:.2e} lse {e_lse:.2e}")


@pytest.mark.parametrize("name", ["gqa_g20_bf16", "mla_h16_b4", "gqa_g12_bf16"])
def test_private_pages_hint(name):
    """Plans told that requests share no page: batches of 16-63 rows per KV
    head take the one-wave ring shape; the result is the same attention."""
    import split_kv_paged_page_amd as sk
    w = small_cases()[name]
    inp = inputs(name, w)
    d = Decode(inp, flags=sk.ATTN_PLAN_PRIVATE_PAGES)
    rows = w.num_q_heads // w.num_kv_heads * w.q_len
    assert d.plan.stage1_waves == 1 or rows >= 64, d.plan.stage1_waves
    say(f"private pages {name}: B={w.batch} rows={rows} waves={d.plan.stage1_waves} run")
    d.run()
    e_out, e_lse = check_against_oracle(d, tol_for(w))
    print(f"{name}: S={d.S} waves={d.plan.stage1_waves} out {e_out:.2e} lse {e_lse:.2e}")


@pytest.mark.parametrize("name,device_lens", [
    ("varlen_drafts", (200, 512, 3, 1000, 0, 2048)),
    ("gqa_bf16_ragged8", (9000, 0, 2999, 6000, 1, 11800, 64, 129)),
    ("gqa_f32_ragged6", (19999, 1000, 1, 300, 12000, 6500)),
    ("d256_g8", (1, 2049, 0))])
def test_lens_plan_with_shorter_device_lengths(name, device_lens):
    """A work-list plan made for the host lengths, run on device lengths
    that are each no longer (the documented precondition): the splits past
    a shorter request's keys are empty and the result is the attention over
    the device lengths."""
    w = small_cases()[name]
    base = inputs(name, w)
    assert all(d <= h for d, h in zip(device_lens, w.context_lens))
    inp = base.with_(context_lens=np.asarray(device_lens, np.int32))
    say(f"lens plan {name}: host {w.context_lens} device {device_lens}")
    d = Decode(inp, lens=True, host_lens=w.context_lens).run()
    assert d.chunk and d.plan.live_splits > 0
    e_out, e_lse = check_against_oracle(d, tol_for(w))
    print(f"{name}: S={d.S} chunk={d.chunk} out {e_out:.2e} lse {e_lse:.2e}")


@pytest.mark.parametrize("name", list(small_cases()))
def test_parity_small(name):
    w = small_cases()[name]
    inp = inputs(name, w)
    say(f"parity_small {name} B={w.batch} ctx={w.context_lens[:4]} seed={w.seed} run")
    d = Decode(inp, num_splits=w.num_splits).run()
    e_out, e_lse = check_against_oracle(d, tol_for(w))
    print(f"{name}: S={d.S} rows/wg={d.plan.rows_per_wg} tiles={d.plan.head_tiles} "
          f"out {e_out:.2e} lse {e_lse:.2e}")


def random_cases(n=48, seed=20261202, max_ctx=2500, max_batch=4, max_splits=39, max_rows=256):
    """Seeded random shapes across the whole interface: dtype and head dims
    (fp32 64/128, bf16 64/128/256, MLA 576/512 aliased), group sizes 1-24,
    q_len 1-33 with and without causal rows, page sizes 1-64, batches of
    1-4 with ragged contexts (empty ones and ones shorter than q_len
    included), and the planner's split count or a forced one."""
    import dataclasses
    rng = np.random.default_rng(seed)
    base = get("gqa_64k")
    cases = {}
    for i in range(n):
        kind = rng.choice(["bf16", "bf16", "bf16", "mla", "f32"])
        if kind == "mla":
            dk, dv, alias, dt, hkv = 576, 512, True, "bf16", 1
            hq = int(rng.integers(1, 41))
            P = int(rng.choice([1, 1, 16, 64]))
        else:
            dk = dv = int(rng.choice([64, 128] if kind == "f32" else [64, 128, 256]))
            alias, dt = False, ("f32" if kind == "f32" else "bf16")
            hkv = int(rng.integers(1, 5))
            hq = hkv * int(rng.integers(1, 25))
            P = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
        q_len = int(rng.choice([1] * 6 + [2, 3, 4, 5, 8, 17, 33]))
        while (hq // hkv) * q_len > max_rows:       # keep the oracle quick
            q_len = max(1, q_len // 2)
        causal = bool(q_len > 1 and rng.random() < 0.8)
        B = int(rng.integers(1, max_batch + 1))
        ctx = rng.integers(1, max_ctx, B)
        ctx[rng.random(B) < 0.15] = 0
        small = rng.random(B) < 0.15
        ctx[small] = rng.integers(1, q_len + 2, int(small.sum()))
        S = int(rng.integers(1, max_splits + 1)) if rng.random() < 0.4 else 0
        need = sum(-(-int(c) // P) for c in ctx)
        w = dataclasses.replace(base, name=f"rand{i}", batch=B, q_len=q_len, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim_qk=dk, head_dim_v=dv, page_size=P, kv_dtype=dt,
                                context_lens=tuple(int(c) for c in ctx), pool_pages=2 * need + 3,
                                v_aliases_k=alias, causal=causal, num_splits=S, seed=1000 + i)
        cases[f"rand{i:02d}"] = w
    return cases


# 48 shapes with short contexts, then 32 with long contexts, bigger batches
# and split counts up to 300
_RANDOM = dict(random_cases(),
               **{k.replace("rand", "long"): v for k, v in
                  random_cases(n=32, seed=20261203, max_ctx=20000, max_batch=8, max_splits=300, max_rows=64).items()})


@pytest.mark.parametrize("name", list(_RANDOM))
def test_parity_random_shapes(name):
    w = _RANDOM[name]
    say(f"random {name}: {w.kv_dtype} B={w.batch} q_len={w.q_len} heads={w.num_q_heads}/{w.num_kv_heads} "
        f"dims={w.head_dim_qk}/{w.head_dim_v} P={w.page_size} causal={w.causal} ctx={w.context_lens} "
        f"S={w.num_splits} run")
    inp = generate(w)
    d = Decode(inp, num_splits=w.num_splits).run()
    e_out, e_lse = check_against_oracle(d, tol_for(w))
    print(f"{name}: S={d.S} rows/wg={d.plan.rows_per_wg} waves={d.plan.stage1_waves} out {e_out:.2e} "
          f"lse {e_lse:.2e}")


@pytest.mark.parametrize("name", ["gqa_64k_s5000", "mla_b4_private", "mla_wide_b4", "varlen_drafts",
                                  "gqa_g4_bf16", "gqa_g12_bf16", "d256_g8", "mla_h4", "gqa_f32_g8", "gqa_d64_bf16"])
@pytest.mark.parametrize("top,q_gain", [(4.0, 1.0), (1.0, 8.0), (3.0, 4.0)])
def test_parity_rising_and_peaked_scores(name, top, q_gain):
    # Keys scaled up along the context (and/or a peaked q) make the running
    # max climb through many blocks, in steps both below and above the lazy
    # rescale slack, so both the hot loop and its rescale exit are checked.
    w = dict(small_cases(), mla_b4_private=scaled("mla_b48", context_lens=(3000, 1, 2100, 4097), prefix_len=0,
                                                  prefix_group=0))[name]
    inp = ramp(inputs(name, w), top, q_gain)
    say(f"rising {name} top={top} q_gain={q_gain}")
    d = Decode(inp, num_splits=w.num_splits).run()
    # fp32: a score is a D-term fp32 dot product whose rounding error is
    # proportional to sum_d |q_d k_d| * scale; the ramp multiplies that sum by
    # up to G = top * q_gain.  An absolute error e in a score is a relative
    # error of about e in its weight, so the output's bound is 1e-5 * G.
    # bf16's 1e-2 covers its own input rounding (2^-9 relative) at every G.
    tol = tol_for(w) * (top * q_gain if w.kv_dtype == "f32" else 1.0)
    check_against_oracle(d, tol)


@pytest.mark.parametrize("name,splits", [("gqa_tiny_f32", (1, 2, 4, 7, 16)),
                                         ("prefill_small_d64", (1, 2, 5)),
                                         ("gqa_64k_s5000", (1, 3, 64, 79, 200, 300)),
                                         ("gqa_g6_bf16", (1, 17, 40)),
                                         ("gqa_f32_g16", (1, 9, 33)),
                                         ("varlen_drafts", (1, 5, 33)),
                                         ("mla_b48_b16", (2, 17))])
def test_parity_forced_splits(name, splits):
    w = small_cases()[name]
    inp = inputs(name, w)
    d = Decode(inp, max_splits=max(splits))
    for S in splits:
        say(f"forced_splits {name} S={S}")
        d.S = S
        d.run(S)
        check_against_oracle(d, tol_for(w), S=S)


@pytest.mark.parametrize("name,extra", [("gqa_64k_s5000", (0, 1, 63, 64, 3000)),
                                        ("drafts_b1", (0, 1, 700)),
                                        ("mla_wide_b1", (0, 65))])
def test_plan_sized_for_longer_contexts(name, extra):
    """A single request whose context is shorter than the plan's longest:
    the kernels guess the plan's length for their first page-table reads
    and must recover when the guess is wrong (and use it when right)."""
    cases = dict(small_cases(), drafts_b1=scaled("varlen_drafts", context_lens=(1500,), seed=26),
                 mla_wide_b1=scaled("mla_wide", context_lens=(2049,), seed=27))
    w = cases[name]
    inp = inputs(name, w)
    L = int(inp.context_lens[0])
    # a page table wide enough for the longest plan (extra entries: page 0)
    cols = -(-(L + max(extra)) // w.page_size)
    pt = np.zeros((1, cols), dtype=np.int32)
    pt[:, :inp.page_table.shape[1]] = inp.page_table
    inp = inp.with_(page_table=pt)
    for e in extra:
        say(f"longer plan {name} ctx={L} plan max={L + e}")
        d = Decode(inp, max_context_len=L + e).run()
        check_against_oracle(d, tol_for(w))


@pytest.mark.parametrize("base,P", [("gqa_64k", P) for P in (1, 2, 4, 8, 32, 128)] +
                         [("varlen_drafts", 4), ("varlen_drafts", 64), ("mla_b48", 4),
                          ("gqa_tiny_f32", 1), ("gqa_tiny_f32", 4), ("gqa_tiny_f32", 64)])
def test_parity_page_sizes(base, P):
    """Every power-of-two page size the page walk's shift/mask serves, on
    each kernel shape (ragged contexts, so pages end part-filled)."""
    kw = dict(prefix_len=0, prefix_group=0) if base == "mla_b48" else {}
    ctx = (300, 1, 777) if base != "varlen_drafts" else (256, 515, 1030)
    w = scaled(base, context_lens=ctx, page_size=P, seed=40 + P, **kw)
    inp = generate(w)
    say(f"page size {base} P={P}")
    d = Decode(inp, num_splits=w.num_splits).run()
    check_against_oracle(d, tol_for(w))


def _strided(kind):
    """Re-lay the cache tensors out with other strides and NaN in every
    element the kernels must not read."""
    def f(t):
        import torch
        out = dict(t)
        for key in ("k_cache", "v_cache"):
            c = t[key]
            if c is None:
                continue
            if kind == "padded":        # token pitch = D + 64 elements
                big = torch.full((*c.shape[:3], c.shape[3] + 64), float("nan"), dtype=c.dtype, device=c.device)
                big[..., :c.shape[3]] = c
                out[key] = big[..., :c.shape[3]]
            else:                       # token-major pages: [pages, P, H_kv, D]
                tm = torch.full((c.shape[0], c.shape[2], c.shape[1], c.shape[3]), float("nan"), dtype=c.dtype,
                                device=c.device)
                tm.copy_(c.permute(0, 2, 1, 3))
                out[key] = tm.permute(0, 2, 1, 3)
        return out
    return f


@pytest.mark.parametrize("name", ["gqa_64k_s5000", "varlen_drafts", "mla_b4_private", "gqa_tiny_f32",
                                  "prefill_small_d64"])
@pytest.mark.parametrize("kind", ["padded", "token_major"])
def test_parity_strided_pools(name, kind):
    """The same cache contents under other element strides (the descriptor
    carries page, head and token strides): a padded token pitch whose padding
    is NaN, and a token-major page layout."""
    cases = dict(small_cases(), mla_b4_private=scaled("mla_b48", context_lens=(3000, 1, 2100, 4097), prefix_len=0,
                                                      prefix_group=0))
    w = cases[name]
    inp = inputs(name, w) if name in small_cases() else generate(w)
    say(f"strided {name} {kind}")
    d = Decode(inp, num_splits=w.num_splits, relayout=_strided(kind)).run()
    check_against_oracle(d, tol_for(w))


def test_empty_contexts_and_splits():
    w = scaled("gqa_64k", context_lens=(0, 5, 64, 65, 0, 130), pool_pages=64, seed=9)
    inp = generate(w)
    say("empty contexts S=4")
    d = Decode(inp, num_splits=4).run()
    check_against_oracle(d, tol_for(w))
    out, lse = d.out_f64(), d.lse_f64()
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(out[4] == 0) and np.all(np.isneginf(lse[4]))


def designated_tokens(inp, S, where, chunk=None):
    """Per request and KV head, one designated key per split: the first or
    the last key every query row of the request can see in that split."""
    w = inp.w
    toks = []
    for b in range(w.batch):
        L = int(inp.context_lens[b])
        n0 = oracle.visible_keys(L, w.q_len, 0, w.causal)
        per_head = []
        for h in range(w.num_kv_heads):
            ts = []
            for (sb, se) in oracle.split_bounds(L, S, chunk=chunk):
                e = min(se, n0)
                if e <= sb:
                    continue
                if where == "first":
                    ts.append(min(sb + h, e - 1))
                else:
                    ts.append(max(e - 1 - h, sb))
            per_head.append(ts)
        toks.append(per_head)
    return toks


@pytest.mark.parametrize("name,lens", [(n, False) for n in (
    "gqa_tiny_f32", "gqa_64k_b3_ragged", "mla_b48_b16", "mla_wide_b4", "varlen_drafts", "mla_h4", "d256_g8",
    "gqa_f32_g16", "gqa_d64_bf16")] + [(n, True) for n in (
    "mla_wide_b4", "varlen_drafts", "d256_g8", "gqa_bf16_ragged8", "gqa_f32_ragged6")])
@pytest.mark.parametrize("where", ["first", "last"])
def test_bitexact_gather_and_boundaries(name, lens, where):
    """One-hot: the designated key of each split scores 2*dims above all
    others, so its weight is exactly 1 and every other weight is 0; each
    split's o_part must then be that key's V row bit for bit.  lens: plans
    made with the batch's lengths (one fixed split length per request)."""
    w = small_cases()[name]
    base = inputs(name, w)
    probe = Decode(base, num_splits=w.num_splits, lens=lens)
    S, chunk = probe.S, probe.chunk
    del probe
    if lens:
        assert chunk, f"{name}: the lens plan kept the split-count rule"
    toks = designated_tokens(base, S, where, chunk)
    inp = designate(base, toks)
    say(f"bitexact {name} lens={lens} {where} S={S} chunk={chunk}")
    d = Decode(inp, num_splits=S if not lens else 0, lens=lens).run()
    assert d.S == S and d.chunk == chunk
    if S == 1:
        d.partials()
    go, gl = d.split_parts()
    g = w.num_q_heads // w.num_kv_heads
    score_dims = w.head_dim_qk - (w.head_dim_v if w.v_aliases_k else 0)
    P = w.page_size
    checked = 0
    for b in range(w.batch):
        L = int(inp.context_lens[b])
        bounds = oracle.split_bounds(L, S, chunk=chunk)
        for kvh in range(w.num_kv_heads):
            for t in toks[b][kvh]:
                s = next(i for i, (sb, se) in enumerate(bounds) if sb <= t < se)
                page, slot = inp.page_table[b, t // P], t % P
                src = inp.k_cache if w.v_aliases_k else inp.v_cache
                vrow = oracle.to_f64(src[page, kvh, slot, :w.head_dim_v], w.kv_dtype)
                for j in range(w.q_len):
                    for hh in range(g):
                        h = kvh * g + hh
                        np.testing.assert_array_equal(go[b, j, h, s], vrow,
                                                      err_msg=f"b={b} kvh={kvh} t={t} split={s} j={j} h={h}")
                        assert abs(gl[b, j, h, s] - score_dims) <= 1e-6 * score_dims
                        checked += 1
    assert checked > 0


def test_bit_identity_of_relabellings():
    """XCD-aware order and physical page placement change no bits (aiter PR
    #4758, Technical Details item 2)."""
    import split_kv_paged_page_amd as sk
    for name in ("gqa_64k_b3_ragged", "mla_b48_b16"):
        w = small_cases()[name]
        inp = inputs(name, w)
        say(f"relabel {name} default")
        a = Decode(inp).run()
        ref_out, ref_lse, ref_ws = a.out.cpu(), a.lse.cpu(), a.used_ws_bits()
        for flags in (sk.ATTN_PLAN_NO_XCD_REMAP,):
            say(f"relabel {name} flags={flags}")
            bdec = Decode(inp, num_splits=a.S, flags=flags).run()
            assert torch.equal(bdec.out.cpu(), ref_out)
            assert torch.equal(bdec.lse.cpu(), ref_lse)
            assert np.array_equal(bdec.used_ws_bits(), ref_ws)
        # physical page permutation with the page table remapped
        rng = np.random.default_rng(5)
        perm = rng.permutation(inp.k_cache.shape[0])
        k2 = np.empty_like(inp.k_cache)
        k2[perm] = inp.k_cache
        v2 = None
        if inp.v_cache is not None:
            v2 = np.empty_like(inp.v_cache)
            v2[perm] = inp.v_cache
        pt2 = perm[inp.page_table].astype(np.int32)
        say(f"relabel {name} page permutation")
        c = Decode(inp.with_(k_cache=k2, v_cache=v2, page_table=pt2), num_splits=a.S).run()
        assert torch.equal(c.out.cpu(), ref_out)
        assert torch.equal(c.lse.cpu(), ref_lse)


def test_run_equals_partials_then_merge_and_is_deterministic():
    w = small_cases()["gqa_64k_s5000"]
    inp = inputs("gqa_64k_s5000", w)
    say("run vs partials+merge")
    d = Decode(inp).run()
    out, lse, ws = d.out.clone(), d.lse.clone(), d.used_ws_bits()
    d.poison()
    d.partials()
    d.merge()
    assert torch.equal(d.out, out) and torch.equal(d.lse, lse) and np.array_equal(d.used_ws_bits(), ws)
    for _ in range(5):
        d.run()
        assert torch.equal(d.out, out) and np.array_equal(d.used_ws_bits(), ws)


@pytest.mark.parametrize("name", ["gqa_tiny_f32", "mla_b48_b16", "varlen_drafts", "gqa_g4_bf16", "gqa_f32_g8"])
def test_single_split_direct_output_matches_merge(name):
    """With one split, run() lets stage 1 write the output itself; the bits
    must equal stage 1 partials followed by the stage-2 merge."""
    w = small_cases()[name]
    inp = inputs(name, w)
    d = Decode(inp, num_splits=1)
    say(f"single split direct {name}")
    d.run(1)
    out, lse = d.out.clone(), d.lse.clone()
    d.poison()
    d.partials(1)
    d.merge(1)
    assert torch.equal(d.out, out) and torch.equal(d.lse, lse)
    check_against_oracle(d, tol_for(w), S=1)


@pytest.mark.parametrize("name,S", [("gqa_tiny_f32", None), ("gqa_64k_s5000", None), ("gqa_64k_s5000", 300),
                                    ("varlen_drafts", None)])
def test_stage2_alone_on_oracle_partials(name, S):
    """Merge oracle partials (rounded to fp32) on the GPU; compare with the
    oracle's float64 merge of the same rounded partials."""
    w = small_cases()[name]
    inp = inputs(name, w)
    d = Decode(inp, num_splits=S or w.num_splits or 9)
    S = d.S
    po, pl = oracle.split_reference(inp, S)
    po32, pl32 = po.astype(np.float32), pl.astype(np.float32)
    import split_kv_paged_page_amd as sk
    o_off, l_off, _ = sk.attn_decode_workspace_layout(d.plan, S)
    d.poison()
    ws = d.ws
    ws[o_off // 4: o_off // 4 + po32.size] = torch.from_numpy(po32.ravel()).cuda()
    ws[l_off // 4: l_off // 4 + pl32.size] = torch.from_numpy(pl32.ravel()).cuda()
    say(f"stage2 alone {name} S={S}")
    d.merge()
    mo, ml = oracle.merge_reference(po32.astype(np.float64), pl32.astype(np.float64))
    tol = 1e-5 if w.kv_dtype == "f32" else 1e-2
    assert row_rel_err(d.out_f64(), mo) <= tol
    assert lse_err(d.lse_f64(), ml) <= 1e-5


@pytest.mark.parametrize("S,Hq,dtype", [(S, Hq, "bf16") for S in (2, 8, 9, 16, 17, 256, 257, 700) for Hq in (2, 4, 16)] +
                         [(S, 128, "bf16") for S in (2, 16, 17, 40, 100)] +
                         [(S, 16, "f32") for S in (16, 17, 700)] + [(2000, 2, "bf16"), (4096, 2, "f32")])
def test_stage2_alone_on_random_partials(S, Hq, dtype):
    """The merge on seeded partials of every kind the split rule can leave:
    split log-sum-exps spread over +-20 (up to 80 apart within one row),
    empty splits (-inf) scattered and in runs, half of one request's rows
    with every split empty.  Split counts on both sides of the lane rule's
    steps (8 splits per lane up to 16 splits, then 16: 8 and 9, 16 and 17) and past
    one register pass of 16 splits per lane at the 64-lane limit (2,000 and
    4,096: two and four passes); 2 to 128 query heads (two requests) take
    the merge through 1 to 64 lanes per output."""
    B, Hkv, D, P = 2, 2, 128, 16
    rng = np.random.default_rng(1000 + S)
    po = rng.standard_normal((B, 1, Hq, S, D))
    pl = rng.uniform(-20.0, 20.0, (B, 1, Hq, S))
    pl[0, 0, 0] += np.linspace(0.0, 40.0, S)
    pl[rng.random(pl.shape) < 0.15] = -np.inf
    pl[0, 0, 1, S // 3:] = -np.inf
    pl[B - 1, 0, Hq // 2:] = -np.inf
    po[np.isneginf(pl)] = 0.0
    po32, pl32 = po.astype(np.float32), pl.astype(np.float32)
    import split_kv_paged_page_amd as sk
    dt = sk.ATTN_BF16 if dtype == "bf16" else sk.ATTN_F32
    strides = (Hkv * P * D, P * D, D)   # a [page][head][token][dim] pool the merge never reads
    desc = sk.make_desc(batch=B, q_len=1, num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=D, head_dim_v=D,
                        page_size=P, max_pages_per_req=S * 64 // P, dtype=dt, causal=0, v_aliases_k=0,
                        num_pages=1, k_strides=strides, v_strides=strides)
    plan = sk.attn_decode_plan(desc, 64 * S, S, 0)
    o_off, l_off, nbytes = sk.attn_decode_workspace_layout(plan, S)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    ws[o_off // 4: o_off // 4 + po32.size] = torch.from_numpy(po32.ravel()).cuda()
    ws[l_off // 4: l_off // 4 + pl32.size] = torch.from_numpy(pl32.ravel()).cuda()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.full((B, 1, Hq, D), float("nan"), dtype=tdt, device="cuda")
    lse = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device="cuda")
    say(f"stage2 random partials S={S} {dtype}")
    sk.attn_decode_merge(plan, S, ws, out, lse)
    torch.cuda.synchronize()
    mo, ml = oracle.merge_reference(po32.astype(np.float64), pl32.astype(np.float64))
    assert row_rel_err(out.to(torch.float64).cpu().numpy(), mo) <= (1e-2 if dtype == "bf16" else 1e-5)
    assert lse_err(lse.double().cpu().numpy(), ml) <= 1e-5


# ---- full sizes, policy split count with the batch's lengths known on the host
# (the launch configuration the benchmark times) ----

FULL = [("gqa_64k", None), ("gqa_64k_d64", None), ("varlen_drafts", None), ("prefill_2048x4_d64", None),
        ("prefill_2048x4_d128", (0, 3)), ("prefill_varlen_d64", None), ("prefill_varlen_d128", None),
        ("mla_b48", (0, 13, 47)),
        ("mla_wide", (0, 63)), ("mla_b48_ctl", (5, 40)), ("mla_b1", None)]


@pytest.mark.parametrize("name,requests", FULL)
def test_parity_full_size_sampled(name, requests):
    w = get(name)
    say(f"full-size {name}: generating inputs")
    inp = generate(w)
    say(f"full-size {name}: run")
    d = Decode(inp, lens=True).run()
    e_out, e_lse = check_against_oracle(d, tol_for(w), requests=requests)
    print(f"{name}: S={d.S} out {e_out:.2e} lse {e_lse:.2e}")
    if requests is not None:
        # every other request: outputs written, finite, lse finite
        assert not torch.isnan(d.out).any() and torch.isfinite(d.lse).all()


@pytest.mark.parametrize("name", ["gqa_64k_s5000", "mla_b48_b16", "varlen_drafts", "prefill_small_d64", "gqa_f32_g8"])
def test_graph_replays_match_eager(name):
    # The calls allocate nothing and never synchronise, so they can be captured
    # in a graph; every replay, with eager work and synchronisations between
    # replays, must give the eager bits (output, log-sum-exp and partials).
    import split_kv_paged_page_amd as sk
    w = small_cases()[name]
    inp = inputs(name, w)
    say(f"graph {name} eager run")
    d = Decode(inp, num_splits=w.num_splits).run()
    e_out, e_lse, e_ws = d.out.clone(), d.lse.clone(), d.used_ws_bits()
    t = d.t
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    d.poison()
    torch.cuda.synchronize()
    say(f"graph {name} capture")
    with torch.cuda.graph(g, stream=s):
        sk.attn_decode_run(d.plan, t["q"], t["k_cache"], d.v, t["page_table"], t["context_lens"],
                           float(inp.scale), d.S, d.out, d.lse, d.ws, stream=s.cuda_stream)
    for r in range(3):
        d.poison()                       # eager work between replays
        torch.cuda.synchronize()
        say(f"graph {name} replay {r}")
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out.view(torch.int16) if d.out.dtype == torch.bfloat16 else d.out.view(torch.int32),
                           e_out.view(torch.int16) if e_out.dtype == torch.bfloat16 else e_out.view(torch.int32)), r
        assert torch.equal(d.lse.view(torch.int32), e_lse.view(torch.int32)), r
        if d.S > 1:
            assert np.array_equal(d.used_ws_bits(), e_ws), r
