"""GPU parity of the shared-prefix plans (attn_decode_plan_prefix /
attn_decode_run_prefix) against the oracle: the output and log-sum-exp of
every row, and every split slot's partial against the oracle's shared-prefix
split rule (the groups' shared keys split by the rule, then each request's
own keys).  Workloads whose requests in groups of G share their first keys
(the same page ids), as in aiter PR #4758's MLA workload (Test Plan)."""

import numpy as np
import pytest

import oracle
import split_kv_paged_page_amd as sk
from tests.gpu_helpers import lse_err, row_rel_err, say, tol_for, upload, validate_inputs
from workloads import generate, get, scaled
from workloads.gen import designate

pytestmark = pytest.mark.gpu


class PrefixDecode:
    """One uploaded problem + shared-prefix plan.  The mechanism tests force
    the shared pass (ATTN_PLAN_SHARED_PASS), which the planner skips for some
    of the small cases."""

    def __init__(self, inp, flags=sk.ATTN_PLAN_SHARED_PASS):
        import torch
        validate_inputs(inp)
        w = inp.w
        self.inp = inp
        self.t = upload(inp, "cuda")
        t = self.t
        self.desc = sk.make_desc_from_tensors(t["q"], t["k_cache"], t["v_cache"], t["page_table"],
                                              head_dim_v=w.head_dim_v, causal=w.causal)
        mx = int(max(inp.context_lens))
        self.plan = sk.attn_decode_plan_prefix(self.desc, mx, w.prefix_group, w.prefix_len, flags)
        self.S = self.plan.num_splits
        self.prefix = self.plan.prefix_len
        self.Sp = self.plan.shared.num_splits if self.prefix else 0
        self.So = self.plan.own.num_splits
        assert self.S == self.Sp + self.So
        self.dtype = torch.float32 if w.kv_dtype == "f32" else torch.bfloat16
        self.ws = torch.empty(self.plan.workspace_bytes // 4, dtype=torch.float32, device="cuda")
        self.out = torch.empty((w.batch, w.q_len, w.num_q_heads, w.head_dim_v), dtype=self.dtype, device="cuda")
        self.lse = torch.empty((w.batch, w.q_len, w.num_q_heads), dtype=torch.float32, device="cuda")

    def run(self):
        import torch
        t = self.t
        self.ws.fill_(float("nan"))
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))
        v = t["k_cache"] if t["v_cache"] is None else t["v_cache"]
        sk.attn_decode_run_prefix(self.plan, t["q"], t["k_cache"], v, t["page_table"], t["context_lens"],
                                  float(self.inp.scale), self.out, self.lse, self.ws)
        torch.cuda.synchronize()
        return self

    def bounds_of(self):
        return lambda L: oracle.prefix_split_bounds(L, self.prefix, self.Sp, self.So)

    def split_parts(self):
        w = self.inp.w
        rows, S = w.batch * w.q_len * w.num_q_heads, self.S
        l_off = -(-rows * S * w.head_dim_v * 4 // 256) * 256
        ws = self.ws.cpu().numpy()
        o = ws[:rows * S * w.head_dim_v].reshape(w.batch, w.q_len, w.num_q_heads, S, w.head_dim_v)
        l_ = ws[l_off // 4: l_off // 4 + rows * S].reshape(w.batch, w.q_len, w.num_q_heads, S)
        return o.astype(np.float64), l_.astype(np.float64)


def cases():
    return {
        # MLA, groups of 8 sharing 700 of 1,000 keys (the batch-48 shape, smaller)
        "mla_b16_p700": scaled("mla_b48", batch=16, context_lens=(1000,) * 16, prefix_len=700, seed=61),
        # ragged own parts, one of them empty (context = prefix)
        "mla_b16_ragged": scaled("mla_b48", context_lens=(512, 513, 700, 2000, 1100, 640, 777, 1999) * 2,
                                 prefix_len=512, seed=62),
        # 128 heads on the latent head: the shared pass holds 2 x 128 rows per group
        "mla_wide_b4_g2": scaled("mla_wide", context_lens=(1500, 2049, 1300, 1700), prefix_group=2, prefix_len=1280,
                                 seed=63),
        # GQA, page size 16, groups of 2 (8-row own pass on the lone wave, 16-row shared pass)
        "gqa_b4_g2": scaled("gqa_64k", context_lens=(3000, 1500, 1025, 5000), prefix_group=2, prefix_len=1024,
                            seed=64),
        # fp32 on the vector ALUs in both passes
        "gqa_f32_b4_g2": scaled("gqa_tiny_f32", context_lens=(700, 300, 260, 999), prefix_group=2,
                                prefix_len=256, num_splits=0, seed=65),
        # causal draft rows: every row sees the whole shared part
        "drafts_g3": scaled("varlen_drafts", context_lens=(600, 700, 1000, 800, 900, 2048), prefix_group=3,
                            prefix_len=512, seed=66),
        # every request exactly the shared keys: the own pass finds none
        "mla_b16_all_shared": scaled("mla_b48", batch=16, context_lens=(700,) * 16, prefix_len=700, seed=68),
        # prefix 0: the own pass alone over every key
        "gqa_b4_p0": scaled("gqa_64k", context_lens=(3000, 1500, 1025, 5000), prefix_group=2, prefix_len=0,
                            seed=67),
        # MLA in groups of 2 (32 rows): the planner keeps the default plan
        "mla_b4_g2": scaled("mla_b48", context_lens=(1000, 900, 1200, 701), prefix_group=2, prefix_len=700,
                            seed=69),
        # groups of one request: nothing to share
        "gqa_b3_g1": scaled("gqa_64k", context_lens=(2000, 1100, 3000), prefix_group=1, prefix_len=1024,
                            seed=70),
    }


def random_prefix_cases(n=24, seed=20261204):
    """Seeded random shared-prefix shapes: bf16 at head dims 64-256 and MLA
    576/512, fp32 at 64 and 128; 1-16 query heads per KV head, q_len 1-5
    with and without causal rows; groups of 1-4 requests, one or two groups;
    page sizes 1-32; prefixes of 0 to about 1,200 keys (whole pages) and own
    parts from none to 1,500 keys, every request holding the prefix plus
    q_len - 1 keys at least."""
    import dataclasses
    rng = np.random.default_rng(seed)
    base = get("gqa_64k")
    out = {}
    for i in range(n):
        kind = rng.choice(["bf16", "bf16", "mla", "f32"])
        if kind == "mla":
            dk, dv, alias, dt, hkv = 576, 512, True, "bf16", 1
            hq = int(rng.integers(1, 33))
            P = int(rng.choice([1, 16]))
        else:
            dk = dv = int(rng.choice([64, 128] if kind == "f32" else [64, 128, 256]))
            alias, dt = False, ("f32" if kind == "f32" else "bf16")
            hkv = int(rng.integers(1, 4))
            hq = hkv * int(rng.integers(1, 17))
            P = int(rng.choice([1, 2, 4, 8, 16, 32]))
        q_len = int(rng.choice([1] * 5 + [2, 4, 5]))
        while (hq // hkv) * q_len > 128:
            q_len = max(1, q_len // 2)
        causal = bool(q_len > 1 and rng.random() < 0.7)
        G = int(rng.integers(1, 5))
        B = G * int(rng.integers(1, 3))
        prefix = P * int(rng.integers(0, 1200 // P + 1))
        own = rng.integers(0, 1500, B)
        own[rng.random(B) < 0.2] = 0
        ctx = tuple(int(prefix + q_len - 1 + o) for o in own)
        w = dataclasses.replace(base, name=f"prand{i}", batch=B, q_len=q_len, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim_qk=dk, head_dim_v=dv, page_size=P, kv_dtype=dt, context_lens=ctx,
                                v_aliases_k=alias, causal=causal, num_splits=0, seed=2000 + i,
                                prefix_group=G, prefix_len=prefix)
        out[f"prand{i:02d}"] = dataclasses.replace(w, pool_pages=2 * w.pages_needed() + 3)
    return out


_RANDOM = random_prefix_cases()


@pytest.mark.parametrize("name", list(_RANDOM))
def test_prefix_parity_random_shapes(name):
    """Every output, log-sum-exp and split slot against the oracle, with the
    shared pass forced (and, where the group is big enough, also chosen)."""
    w = _RANDOM[name]
    say(f"prefix random {name}: {w.kv_dtype} B={w.batch} G={w.prefix_group} prefix={w.prefix_len} "
        f"q_len={w.q_len} heads={w.num_q_heads}/{w.num_kv_heads} dims={w.head_dim_qk}/{w.head_dim_v} "
        f"P={w.page_size} causal={w.causal} ctx={w.context_lens}")
    d = PrefixDecode(generate(w))
    say(f"  S = {d.Sp} + {d.So}")
    e = check(d.run())
    say(f"  out {e[0]:.2e} lse {e[1]:.2e}")


_INPUTS = {}


def inputs(name):
    if name not in _INPUTS:
        _INPUTS[name] = generate(cases()[name])
    return _INPUTS[name]


def check(d: PrefixDecode, requests=None):
    inp, w = d.inp, d.inp.w
    ro, rl = oracle.decode_reference(inp, requests=requests)
    sel = slice(None) if requests is None else list(requests)
    tol = tol_for(w)
    e_out = row_rel_err(d.out.double().cpu().numpy()[sel], ro[sel])
    e_lse = lse_err(d.lse.double().cpu().numpy()[sel], rl[sel])
    assert e_out <= tol, f"output rel err {e_out:.3e} > {tol}"
    assert e_lse <= 1e-3, f"lse err {e_lse:.3e}"
    po, pl = oracle.split_reference(inp, d.S, requests=requests, bounds_of=d.bounds_of())
    go, gl = d.split_parts()
    e_po = row_rel_err(go[sel], po[sel])
    e_pl = lse_err(gl[sel], pl[sel])
    assert e_po <= tol, f"partials rel err {e_po:.3e}"
    assert e_pl <= 1e-3, f"partial lse err {e_pl:.3e}"
    return e_out, e_lse


@pytest.mark.parametrize("name", list(cases()))
def test_prefix_parity_small(name):
    d = PrefixDecode(inputs(name))
    say(f"prefix {name} S = {d.Sp} + {d.So}")
    e = check(d.run())
    say(f"  out {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("name", ["mla_b16_p700", "gqa_b4_g2", "gqa_f32_b4_g2", "drafts_g3"])
def test_prefix_matches_the_plain_plan(name):
    """The same inputs through attn_decode_run: equal within the tolerance
    (the split sets differ, so the rounding does)."""
    import torch
    inp = inputs(name)
    d = PrefixDecode(inp).run()
    t = d.t
    v = t["k_cache"] if t["v_cache"] is None else t["v_cache"]
    plan = sk.attn_decode_plan(d.desc, int(max(inp.context_lens)))
    ws = torch.empty(plan.workspace_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    out = torch.empty_like(d.out)
    lse = torch.empty_like(d.lse)
    sk.attn_decode_run(plan, t["q"], t["k_cache"], v, t["page_table"], t["context_lens"], float(inp.scale), 0,
                       out, lse, ws)
    torch.cuda.synchronize()
    assert row_rel_err(d.out.double().cpu().numpy(), out.double().cpu().numpy()) <= tol_for(inp.w)
    assert lse_err(d.lse.double().cpu().numpy(), lse.double().cpu().numpy()) <= 1e-3


@pytest.mark.parametrize("where", ["first", "last"])
@pytest.mark.parametrize("name", ["mla_b16_ragged", "gqa_b4_g2", "drafts_g3"])
def test_prefix_bitexact_gather_and_boundaries(name, where):
    """One-hot keys at the first (or last) key of every split slot of every
    request, shared slots included: each slot's partial must be that key's V
    row bit for bit, which shows that the shared pass read the group's pages
    and that every slot covers exactly its range."""
    base = inputs(name)
    w = base.w
    probe = PrefixDecode(base)
    bounds_of = probe.bounds_of()
    del probe
    toks = []
    for b in range(w.batch):
        L = int(base.context_lens[b])
        n0 = oracle.visible_keys(L, w.q_len, 0, w.causal)
        per_head = []
        for h in range(w.num_kv_heads):
            ts = []
            for (sb, se) in bounds_of(L):
                e = min(se, n0)
                if e <= sb:
                    continue
                ts.append(min(sb + h, e - 1) if where == "first" else max(e - 1 - h, sb))
            per_head.append(ts)
        toks.append(per_head)
    inp = designate(base, toks)
    d = PrefixDecode(inp).run()
    go, gl = d.split_parts()
    g = w.num_q_heads // w.num_kv_heads
    score_dims = w.head_dim_qk - (w.head_dim_v if w.v_aliases_k else 0)
    checked = 0
    for b in range(w.batch):
        L = int(inp.context_lens[b])
        bounds = bounds_of(L)
        for kvh in range(w.num_kv_heads):
            for t in toks[b][kvh]:
                s = next(i for i, (sb, se) in enumerate(bounds) if sb <= t < se)
                page, slot = inp.page_table[b, t // w.page_size], t % w.page_size
                src = inp.k_cache if w.v_aliases_k else inp.v_cache
                vrow = oracle.to_f64(src[page, kvh, slot, :w.head_dim_v], w.kv_dtype)
                for j in range(w.q_len):
                    for hh in range(g):
                        h = kvh * g + hh
                        np.testing.assert_array_equal(go[b, j, h, s], vrow, err_msg=f"b={b} t={t} s={s} h={h}")
                        assert abs(gl[b, j, h, s] - score_dims) <= 1e-6 * score_dims
                        checked += 1
    assert checked > 0


def test_prefix_full_size_mla_b48_sampled():
    """The MLA batch-48 workload itself (groups of 8 sharing 63,240 of 68,000
    keys), sampled requests from three groups against the oracle."""
    inp = generate(get("mla_b48"))
    d = PrefixDecode(inp).run()
    say(f"prefix mla_b48 S = {d.Sp} + {d.So}")
    check(d, requests=(0, 9, 47))


@pytest.mark.parametrize("name,falls_back", [("mla_b4_g2", True), ("gqa_b3_g1", True), ("gqa_b4_g2", True),
                                              ("drafts_g3", False), ("mla_b16_p700", False),
                                              ("mla_wide_b4_g2", False)])
def test_prefix_fallback_is_the_plain_run(name, falls_back):
    """Without ATTN_PLAN_SHARED_PASS: where the planner keeps the default plan
    (MLA in groups of 2, groups of one request, GQA groups of 16 rows)
    attn_decode_run_prefix gives attn_decode_run's bits; elsewhere the
    shared pass runs and matches the oracle."""
    import torch
    inp = inputs(name)
    d = PrefixDecode(inp, flags=0).run()
    say(f"prefix fallback {name}: S = {d.Sp} + {d.So}")
    check(d)
    if not falls_back:
        assert d.prefix == inp.w.prefix_len and d.Sp > 0
        return
    assert d.prefix == 0 and d.Sp == 0
    t = d.t
    v = t["k_cache"] if t["v_cache"] is None else t["v_cache"]
    plan = sk.attn_decode_plan(d.desc, int(max(inp.context_lens)))
    assert plan.key == d.plan.own.key and plan.num_splits == d.S
    ws = torch.empty(plan.workspace_bytes // 4, dtype=torch.float32, device="cuda")
    out = torch.empty_like(d.out)
    lse = torch.empty_like(d.lse)
    sk.attn_decode_run(plan, t["q"], t["k_cache"], v, t["page_table"], t["context_lens"], float(inp.scale), 0,
                       out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(d.out.view(torch.int16), out.view(torch.int16))
    assert torch.equal(d.lse.view(torch.int32), lse.view(torch.int32))


def test_prefix_full_size_gqa_b8_shared_sampled():
    """Eight 64K-key GQA requests sharing 61,440 keys: the shared-prefix plan
    (which the planner takes for this group) and the default plan (two
    one-wave workgroups per CU), sampled requests against the oracle."""
    import torch
    inp = generate(get("gqa_64k_b8_shared"))
    d = PrefixDecode(inp, flags=0).run()
    say(f"prefix gqa_64k_b8_shared S = {d.Sp} + {d.So}")
    assert d.prefix == 61440 and d.Sp > 0
    check(d, requests=(0, 5))
    t = d.t
    plan = sk.attn_decode_plan(d.desc, 65536)
    ws = torch.empty(plan.workspace_bytes // 4, dtype=torch.float32, device="cuda")
    out = torch.empty_like(d.out)
    lse = torch.empty_like(d.lse)
    sk.attn_decode_run(plan, t["q"], t["k_cache"], t["v_cache"], t["page_table"], t["context_lens"],
                       float(inp.scale), 0, out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_reference(inp, requests=(0, 5))
    sel = [0, 5]
    assert row_rel_err(out.double().cpu().numpy()[sel], ro[sel]) <= tol_for(inp.w)
    assert lse_err(lse.double().cpu().numpy()[sel], rl[sel]) <= 1e-3


@pytest.mark.parametrize("name", ["mla_b16_p700", "gqa_b4_g2"])
def test_prefix_graph_replays_match_eager(name):
    """attn_decode_run_prefix allocates nothing and never synchronises: its
    three launches captured in a graph give the eager bits on every replay,
    with eager work and synchronisations between replays."""
    import torch
    d = PrefixDecode(inputs(name)).run()
    e_out, e_lse = d.out.clone(), d.lse.clone()
    e_ws = d.ws.clone()
    t = d.t
    v = t["k_cache"] if t["v_cache"] is None else t["v_cache"]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        sk.attn_decode_run_prefix(d.plan, t["q"], t["k_cache"], v, t["page_table"], t["context_lens"],
                                  float(d.inp.scale), d.out, d.lse, d.ws, stream=s.cuda_stream)
    for r in range(3):
        d.ws.fill_(float("nan"))          # eager work between replays
        d.out.fill_(float("nan"))
        d.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"prefix graph {name} replay {r}")
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out.view(torch.int16), e_out.view(torch.int16)), r
        assert torch.equal(d.lse.view(torch.int32), e_lse.view(torch.int32)), r
        w = d.inp.w
        rows = w.batch * w.q_len * w.num_q_heads
        n_o = rows * d.S * w.head_dim_v
        l_off = -(-n_o * 4 // 256) * 256 // 4
        assert torch.equal(d.ws[:n_o].view(torch.int32), e_ws[:n_o].view(torch.int32)), r
        assert torch.equal(d.ws[l_off:l_off + rows * d.S].view(torch.int32),
                           e_ws[l_off:l_off + rows * d.S].view(torch.int32)), r
