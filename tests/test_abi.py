"""The C ABI on the host (no GPU): the library loads and exports every
function include/attn_decode.h declares, the ctypes structs match the C
layout, the planner's split rule equals the oracle's, the P2 policy mode
reproduces the split counts of aiter PR #4758's Test Result table 1, plan
keys cover every shape field, and invalid arguments come back as status
codes with a message (no kernel is launched on any of these paths)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import split_kv_paged_page_amd as sk
from tests.test_oracle import read_table

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_decode.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:attn_status|const char\*)\s+(attn_\w+)\s*\(", txt, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 7
    L = sk.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(sk.EXPORTED) == names
    out = subprocess.run(["nm", "-D", "--defined-only", sk.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, re.M), n


def test_struct_layout_matches_header(tmp_path):
    fields_d = [f for f, _ in sk.AttnDecodeDesc._fields_]
    fields_p = [f for f, _ in sk.AttnDecodePlan._fields_]
    fields_pp = [f for f, _ in sk.AttnDecodePrefixPlan._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void){",
           'printf("%zu %zu %zu\\n", sizeof(attn_decode_desc), sizeof(attn_decode_plan_t), '
           'sizeof(attn_decode_prefix_plan_t));']
    for f in fields_pp:
        src.append(f'printf("x {f} %zu\\n", offsetof(attn_decode_prefix_plan_t, {f}));')
    for f in fields_d:
        src.append(f'printf("d {f} %zu\\n", offsetof(attn_decode_desc, {f}));')
    for f in fields_p:
        src.append(f'printf("p {f} %zu\\n", offsetof(attn_decode_plan_t, {f}));')
    src.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(c), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    sd, sp, spp = map(int, lines[0].split())
    assert sd == ctypes.sizeof(sk.AttnDecodeDesc) and sp == ctypes.sizeof(sk.AttnDecodePlan)
    assert spp == ctypes.sizeof(sk.AttnDecodePrefixPlan)
    for ln in lines[1:]:
        if not ln:
            continue
        kind, f, off = ln.split()
        cls = {"d": sk.AttnDecodeDesc, "p": sk.AttnDecodePlan, "x": sk.AttnDecodePrefixPlan}[kind]
        assert getattr(cls, f).offset == int(off), (kind, f)


def desc(B=1, q_len=1, Hq=16, Hkv=2, Dk=128, Dv=128, P=16, maxp=4096, dtype=sk.ATTN_BF16, causal=0,
         alias=0, pages=8192):
    ks = (Hkv * P * Dk, P * Dk, Dk)
    vs = ks if alias else (Hkv * P * Dv, P * Dv, Dv)
    return sk.make_desc(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=Dk,
                        head_dim_v=Dv, page_size=P, max_pages_per_req=maxp, dtype=dtype, causal=causal,
                        v_aliases_k=alias, num_pages=pages, k_strides=ks, v_strides=vs)


def mla_desc(B):
    return desc(B=B, Hq=16, Hkv=1, Dk=576, Dv=512, P=1, maxp=68000, alias=1, pages=655360)


def test_plan_split_rule_equals_oracle():
    rng = np.random.default_rng(0)
    p = sk.attn_decode_plan(desc(), 65536, 0)
    for L in list(range(0, 300)) + list(rng.integers(0, 65536, 300)):
        for S in (1, 2, 3, 5, 7, 64, 128, 333):
            ref = oracle.split_bounds(int(L), S, 64)
            for s in range(S):
                assert sk.attn_decode_split_range(p, int(L), S, s) == ref[s]


def test_p2_policy_reproduces_table():
    ctx, rows = read_table("aiter4758_policy_table.txt")
    for r in rows:
        p = sk.attn_decode_plan(mla_desc(r["conc"]), ctx, 0, sk.ATTN_PLAN_POLICY_P2)
        assert p.num_splits == r["splits"], r
        b, e = sk.attn_decode_split_range(p, ctx, 0, 0)
        assert (e - b) // 64 == r["trips"] and (e - b) % 64 == 0


def test_default_split_count_leaves_no_split_empty_at_the_longest_context():
    rng = np.random.default_rng(5)
    for _ in range(200):
        B, hkv = int(rng.integers(1, 9)), int(rng.choice([1, 2, 4, 8]))
        L = int(rng.integers(1, 200000))
        p = sk.attn_decode_plan(desc(B=B, Hq=hkv * int(rng.integers(1, 9)), Hkv=hkv, maxp=(L + 15) // 16), L, 0)
        b, e = sk.attn_decode_split_range(p, L, 0, p.num_splits - 1)
        assert e > b, (B, hkv, L, p.num_splits)        # the last split holds keys


def test_default_policy_fills_the_chip():
    p = sk.attn_decode_plan(desc(), 65536, 0)
    wgs = p.num_splits * 1 * 2 * p.head_tiles
    assert wgs >= 256
    p = sk.attn_decode_plan(desc(), 100, 0)      # short context: never more splits than 64-key blocks
    assert p.num_splits == 2


def test_workgroups_per_cu_of_the_one_wave_ring():
    """The one-wave ring at head dim 128 runs one workgroup per CU for one
    request or a batch with the private-pages hint, and two for a batch whose
    requests may share pages; at head dim 64 two, and four for such a batch."""
    priv = sk.ATTN_PLAN_PRIVATE_PAGES
    S = lambda d, f=0: sk.attn_decode_plan(d, 65536, 0, f).num_splits
    assert S(desc(B=1)) == 128 and S(desc(B=1), priv) == 128          # 256 / (1 x 2 KV heads)
    assert S(desc(B=4)) == 64 and S(desc(B=4), priv) == 32             # 512 or 256 / (4 x 2)
    assert S(desc(B=8)) == 32 and S(desc(B=8), priv) == 16
    d64 = dict(Dk=64, Dv=64)
    assert S(desc(B=1, **d64)) == 256 and S(desc(B=4, **d64), priv) == 64
    assert S(desc(B=4, **d64)) == 128 and S(desc(B=8, **d64)) == 64     # 1024 / (B x 2)


def test_kernel_choice_by_rows_per_kv_head():
    # (query heads, KV heads, q_len, head dims, dtype) -> (variant, rows per workgroup, waves)
    V, M = sk.ATTN_VARIANT_VALU, sk.ATTN_VARIANT_MFMA
    F32 = sk.ATTN_F32
    cases = [
        (dict(Hq=2), (M, 16, 1)),                         # 1 row: one wave on a ring, tile mostly empty
        (dict(Hq=8), (M, 16, 1)),                         # 4 rows
        (dict(Hq=16), (M, 16, 1)),                        # 8 rows
        (dict(Hq=24), (M, 16, 1)),                        # 12 rows
        (dict(Hq=32), (M, 16, 4)),                        # 16 rows: four key streams
        (dict(Hq=40), (M, 16, 4)),                        # 20 rows: two head tiles
        (dict(Hq=64, Hkv=8, q_len=4, Dk=256, Dv=256, causal=1), (M, 32, 2)),   # 32 draft rows
        (dict(Hq=16, Hkv=2, Dk=256, Dv=256), (M, 16, 1)), # 8 rows at head dim 256
        (dict(Hq=8, dtype=F32), (V, 4, 4)),               # fp32 stays on the vector ALUs
        (dict(Hq=16, dtype=F32), (V, 8, 4)),
        (dict(Hq=32, dtype=F32), (V, 8, 4)),              # 16 rows: two 8-row tiles at head dim 128
        (dict(Hq=4, Hkv=1, Dk=64, Dv=64, dtype=F32), (V, 4, 4)),
    ]
    for kw, want in cases:
        p = sk.attn_decode_plan(desc(B=4, **kw), 4096, 0)
        assert (p.variant, p.rows_per_wg, p.stage1_waves) == want, (kw, want)
        # one request: the ring shapes instead of key streams (one wave per 16-row tile)
        p1 = sk.attn_decode_plan(desc(B=1, **kw), 4096, 0)
        want1 = (M, 16, 1) if want[0] == M and want[2] == 4 and want[1] == 16 else want
        assert (p1.variant, p1.rows_per_wg, p1.stage1_waves) == want1, (kw, want1)
    mla = dict(Hkv=1, Dk=576, Dv=512, P=1, maxp=68000, alias=1, pages=655360)
    for hq, want in ((4, (M, 16, 1)), (16, (M, 16, 4)), (128, (M, 64, 4))):
        p = sk.attn_decode_plan(desc(B=48, Hq=hq, **mla), 68000, 0)
        assert (p.variant, p.rows_per_wg, p.stage1_waves) == want, (hq, want)
    assert sk.attn_decode_plan(desc(B=1, Hq=16, **mla), 68000, 0).stage1_waves == 1
    # requests that share no page (the caller's hint): the ring shape for a batch too
    priv = sk.ATTN_PLAN_PRIVATE_PAGES
    assert sk.attn_decode_plan(desc(B=48, Hq=16, **mla), 68000, 0, priv).stage1_waves == 1
    assert sk.attn_decode_plan(desc(B=4, Hq=32), 4096, 0, priv).stage1_waves == 1
    assert sk.attn_decode_plan(desc(B=4, Hq=128, Hkv=2), 4096, 0, priv).stage1_waves == 4   # 64 rows: a ring already
    assert sk.attn_decode_plan(desc(B=4, Hq=32), 4096, 0, priv).key != sk.attn_decode_plan(desc(B=4, Hq=32), 4096, 0).key
    with pytest.raises(sk.AttnDecodeError) as ei:      # unknown flag bits
        sk.attn_decode_plan(desc(B=4), 4096, 0, 16)
    assert ei.value.status == sk.ATTN_EINVAL
    assert sk.attn_decode_plan(desc(Hq=16, Dk=64, Dv=64), 4096, 0).variant == M     # bf16 head dim 64
    # causal prefill rows (query positions x group) at head dims 64 and 128: four 16-row waves sharing
    # each block from 64 rows on (eight from 128 at head dim 128), four key streams from 16
    for d in (64, 128):
        wide = (M, 128, 8) if d == 128 else (M, 64, 4)
        for q_len, want in ((4, (M, 16, 4)), (15, (M, 16, 4)), (16, (M, 64, 4)), (2048, wide)):
            p = sk.attn_decode_plan(desc(B=4, Hq=16, Hkv=4, q_len=q_len, Dk=d, Dv=d, causal=1), 4096, 0)
            assert (p.variant, p.rows_per_wg, p.stage1_waves) == want, (d, q_len, want)
    with pytest.raises(sk.AttnDecodeError):      # no kernel at head dim 96
        sk.attn_decode_plan(desc(Hq=16, Dk=96, Dv=96), 4096, 0)


def test_default_split_count_fills_one_round():
    # two workgroups per CU where the LDS allows (vector-ALU kernel, the lone
    # matrix-core wave at head dim 64), one otherwise (and for the lone wave at
    # head dim 128, whose two blocks in flight keep a CU streaming)
    assert sk.attn_decode_plan(desc(), 65536, 0).num_splits == 256 // 2
    assert sk.attn_decode_plan(desc(Dk=64, Dv=64), 65536, 0).num_splits == 512 // 2
    assert sk.attn_decode_plan(desc(dtype=sk.ATTN_F32), 65536, 0).num_splits == 512 // 2
    mla = dict(Hkv=1, Dk=576, Dv=512, P=1, maxp=68000, alias=1, pages=655360)
    assert sk.attn_decode_plan(desc(B=48, Hq=4, **mla), 68000, 0).num_splits == 256 // 48
    assert sk.attn_decode_plan(desc(B=48, Hq=16, **mla), 68000, 0).num_splits == 256 // 48
    # drafts: one round would be 256 // 24 = 10 splits, but 2,048 keys in 256-key chunks fill only 8
    assert sk.attn_decode_plan(desc(B=6, Hq=32, Hkv=4, Dk=256, Dv=256), 2048, 0).num_splits == 8


def test_plan_key_covers_shape_fields():
    # rocm-libraries PR #10102, Technical Details: two configurations that differ only in
    # batch shared a launcher-cache entry; every descriptor field must reach the key.
    base = sk.attn_decode_plan(desc(B=4, maxp=2048), 2048, 8).key
    keys = {base}
    for kw in (dict(B=6), dict(maxp=2049), dict(Hq=32), dict(P=32, maxp=1024), dict(causal=1),
               dict(pages=9000), dict(dtype=sk.ATTN_F32)):
        args = dict(B=4, maxp=2048)
        args.update(kw)
        if args.get("dtype") == sk.ATTN_F32:
            args.update(Dk=128, Dv=128)
        k = sk.attn_decode_plan(desc(**args), 2048, 8).key
        assert k not in keys, kw
        keys.add(k)
    assert sk.attn_decode_plan(desc(B=4, maxp=2048), 2048, 16).key != base
    assert sk.attn_decode_plan(desc(B=4, maxp=2048), 2048, 8, sk.ATTN_PLAN_NO_XCD_REMAP).key != base
    assert sk.attn_decode_plan(desc(B=4, maxp=2048), 2048, 8).key == base


def test_workspace_layout():
    p = sk.attn_decode_plan(desc(), 65536, 128)
    o, l_, b = sk.attn_decode_workspace_layout(p, 0)
    rows = 16
    assert o == 0 and l_ == rows * 128 * 128 * 4 and b >= l_ + rows * 128 * 4 and b == p.workspace_bytes
    _, _, b64 = sk.attn_decode_workspace_layout(p, 64)
    assert b64 < b


def test_fused_merge_plan_layout_and_init_checks():
    # The in-kernel merge keeps one counter per (request, KV head, head tile)
    # at the workspace's start; o_part and lse_part move up by that block.
    plain = sk.attn_decode_plan(desc(B=3), 4096, 8)
    fused = sk.attn_decode_plan(desc(B=3), 4096, 8, sk.ATTN_PLAN_FUSED_MERGE)
    assert fused.key != plain.key and fused.variant == sk.ATTN_VARIANT_MFMA
    counters = 3 * 2 * fused.head_tiles
    shift = (counters * 4 + 255) // 256 * 256
    for S in (0, 2, 5):
        po, pl_, pb = sk.attn_decode_workspace_layout(plain, S)
        fo, fl, fb = sk.attn_decode_workspace_layout(fused, S)
        assert (fo, fl, fb) == (po + shift, pl_ + shift, pb + shift)
    assert fused.workspace_bytes == plain.workspace_bytes + shift
    # two head tiles of 16 rows (20 rows per KV head): counters per tile
    two = sk.attn_decode_plan(desc(B=2, Hq=40, Hkv=2), 4096, 4, sk.ATTN_PLAN_FUSED_MERGE)
    assert two.head_tiles == 2 and sk.attn_decode_workspace_layout(two, 0)[0] == 256
    # fp32 runs on the vector ALUs, which have no in-kernel merge
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_plan(desc(dtype=sk.ATTN_F32), 4096, 8, sk.ATTN_PLAN_FUSED_MERGE)
    assert ei.value.status == sk.ATTN_EUNSUPPORTED
    # init: nothing to do without the flag; argument errors before any launch
    sk.attn_decode_workspace_init(plain, None, 0, stream=0)
    L = sk.lib()
    assert L.attn_decode_workspace_init(ctypes.byref(fused), None, 1 << 20, None) == sk.ATTN_EINVAL
    assert L.attn_decode_workspace_init(ctypes.byref(fused), (1 << 20) + 16, 1 << 20, None) == sk.ATTN_EINVAL
    assert L.attn_decode_workspace_init(ctypes.byref(fused), 1 << 20, counters * 4 - 4, None) == sk.ATTN_EWORKSPACE
    with pytest.raises(sk.AttnDecodeError) as ei:      # an unknown flag bit
        sk.attn_decode_plan(desc(), 4096, 8, 16)
    assert ei.value.status == sk.ATTN_EINVAL


@pytest.mark.parametrize("mutate,status", [
    (dict(Hq=15), sk.ATTN_EINVAL),
    (dict(B=0), sk.ATTN_EINVAL),
    (dict(Dk=96, Dv=96), sk.ATTN_EUNSUPPORTED),
    (dict(dtype=7), sk.ATTN_EINVAL),
    (dict(alias=1, Dv=256), sk.ATTN_EINVAL),
])
def test_plan_rejects(mutate, status):
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_plan(desc(**mutate), 1024, 0)
    assert ei.value.status == status
    assert sk.attn_decode_last_error()


def test_plan_rejects_page_size_not_power_of_two():
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_plan(desc(P=24, maxp=100), 1024, 0)
    assert ei.value.status == sk.ATTN_EUNSUPPORTED


def test_plan_rejects_index_ranges_past_31_bits():
    # the kernels divide context lengths and row indices as 31-bit values
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_plan(desc(P=1, maxp=(1 << 30) + 1), 1024, 0)
    assert ei.value.status == sk.ATTN_EINVAL
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_plan(desc(B=1 << 20, Hq=512, Hkv=1, maxp=64), 1024, 0)
    assert ei.value.status == sk.ATTN_EINVAL
    sk.attn_decode_plan(desc(P=1, maxp=1 << 30), 1024, 0)


def test_plan_rejects_misaligned_stride():
    d = desc()
    d.k_stride_tok = 129          # 258-byte rows break 16-byte alignment
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_plan(d, 1024, 0)
    assert ei.value.status == sk.ATTN_EUNSUPPORTED


def test_plan_rejects_context_beyond_page_table():
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_plan(desc(maxp=10), 161, 0)
    assert ei.value.status == sk.ATTN_EINVAL


def test_run_argument_errors_before_any_launch():
    p = sk.attn_decode_plan(desc(), 65536, 8)
    fake = 1 << 20  # never dereferenced: validation fails first
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run(p, fake, fake, fake, fake, fake, 0.1, 9, fake, None, fake, 1 << 30, stream=0)
    assert ei.value.status == sk.ATTN_EWORKSPACE
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run(p, None, fake, fake, fake, fake, 0.1, 0, fake, None, fake, 1 << 30, stream=0)
    assert ei.value.status == sk.ATTN_EINVAL
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run(p, fake, fake, fake, fake, fake, 0.1, 0, fake, None, fake, 16, stream=0)
    assert ei.value.status == sk.ATTN_EWORKSPACE
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run(p, fake + 8, fake, fake, fake, fake, 0.1, 0, fake, None, fake, 1 << 30, stream=0)
    assert ei.value.status == sk.ATTN_EINVAL
    # scale must be positive and finite (the kernels scale the block maximum, not each score)
    for bad in (float("nan"), 0.0, -0.1, float("inf"), 3.0e38):
        for call in (sk.attn_decode_run, sk.attn_decode_partials):
            args = (p, fake, fake, fake, fake, fake, bad, 0)
            with pytest.raises(sk.AttnDecodeError) as ei:
                if call is sk.attn_decode_run:
                    call(*args, fake, None, fake, 1 << 30, stream=0)
                else:
                    call(*args, fake, 1 << 30, stream=0)
            assert ei.value.status == sk.ATTN_EINVAL, bad


def test_prefix_plan_passes_and_split_rule():
    """MLA batch 48 with 8-request groups sharing 63,240 keys: the shared pass
    is one 128-row request per group (two 64-row head tiles) over the prefix,
    the own pass every request over its private keys with the private-pages
    hint; the row's slots are the shared splits then the own ones, by the
    oracle's shared-prefix split rule."""
    d = mla_desc(48)
    pp = sk.attn_decode_plan_prefix(d, 68000, 8, 63240)
    sh, own = pp.shared, pp.own
    assert (sh.desc.batch, sh.desc.q_len, sh.desc.causal) == (6, 8, 0)
    assert sh.max_context_len == 63240 and own.max_context_len == 68000 - 63240
    assert sh.variant == sk.ATTN_VARIANT_MFMA and sh.rows_per_wg * sh.head_tiles >= 128
    assert sh.xcd_remap == 1
    assert own.flags & sk.ATTN_PLAN_PRIVATE_PAGES
    assert pp.num_splits == sh.num_splits + own.num_splits
    # one round of workgroups in each pass
    assert 0 < 6 * sh.head_tiles * sh.num_splits <= 512
    assert 0 < 48 * own.head_tiles * own.num_splits <= 512
    al = lambda x: -(-x // 256) * 256
    rows, S = 48 * 16, pp.num_splits
    assert pp.workspace_bytes == al(rows * S * 512 * 4) + al(rows * S * 4)
    for L in (63240, 63241, 64000, 68000):
        got = [sk.attn_decode_split_range(sh, 63240, sh.num_splits, s) for s in range(sh.num_splits)]
        got += [tuple(63240 + x for x in sk.attn_decode_split_range(own, L - 63240, own.num_splits, s))
                for s in range(own.num_splits)]
        assert got == oracle.prefix_split_bounds(L, 63240, sh.num_splits, own.num_splits)
    # keys differ with the grouping and the prefix
    assert sk.attn_decode_plan_prefix(d, 68000, 8, 63000).key != pp.key
    assert sk.attn_decode_plan_prefix(d, 68000, 4, 63240).key != pp.key
    # no prefix: the own pass alone
    p0 = sk.attn_decode_plan_prefix(d, 68000, 8, 0)
    assert p0.shared.num_splits == 0 and p0.num_splits == p0.own.num_splits


def test_prefix_plan_falls_back_where_the_shared_pass_does_not_pay():
    """Without ATTN_PLAN_SHARED_PASS the plan is the default plan over every
    key for groups of one request, for fewer than 32 rows per group and KV
    head, for a single group of fewer than 64, and where the default plan
    runs four key streams (16-63 rows per KV head) with fewer than
    SHARED_PASS_MIN_ROWS rows per group; the caller's other flags reach that
    plan."""
    assert sk.SHARED_PASS_MIN_ROWS == 128

    def check_fallback(d, mx, G, prefix, flags=0):
        pp = sk.attn_decode_plan_prefix(d, mx, G, prefix, flags)
        plain = sk.attn_decode_plan(d, mx, 0, flags)
        assert pp.prefix_len == 0 and pp.shared.num_splits == 0 and pp.prefix_group == G
        assert pp.own.key == plain.key and pp.num_splits == plain.num_splits
        assert pp.workspace_bytes == plain.workspace_bytes
        forced = sk.attn_decode_plan_prefix(d, mx, G, prefix, flags | sk.ATTN_PLAN_SHARED_PASS)
        assert forced.prefix_len == prefix and forced.shared.num_splits > 0 and forced.key != pp.key
        assert not (forced.own.flags & sk.ATTN_PLAN_SHARED_PASS)
        return pp

    def shared(d, mx, G, prefix):
        pp = sk.attn_decode_plan_prefix(d, mx, G, prefix)
        assert pp.prefix_len == prefix and pp.shared.num_splits > 0
        return pp

    # MLA, 16 heads: the default plan runs key streams; 16, 32, 64 rows fall
    # back, 8 requests (128 rows) share
    d = mla_desc(48)
    assert sk.attn_decode_plan(d, 68000).stage1_waves == 4 and sk.attn_decode_plan(d, 68000).rows_per_wg == 16
    for G in (1, 2, 4):
        check_fallback(d, 68000, G, 63240)
    shared(d, 68000, 8, 63240)
    # the caller's flags reach the fallback plan
    nr = check_fallback(d, 68000, 4, 63240, sk.ATTN_PLAN_NO_XCD_REMAP)
    assert nr.own.flags == sk.ATTN_PLAN_NO_XCD_REMAP and nr.own.xcd_remap == 0
    # with the private-pages hint the default plan is the one-wave ring: shared
    pv = sk.attn_decode_plan_prefix(d, 68000, 4, 63240, sk.ATTN_PLAN_PRIVATE_PAGES)
    assert pv.prefix_len == 63240
    # GQA, 8 heads per KV head (the one-wave ring): groups of 2 (16 rows)
    # fall back; groups of 4 (32 rows) share unless they are the only group;
    # groups of 8 and 16 share; a group of one never does
    g = desc(B=16)
    assert sk.attn_decode_plan(g, 65536).stage1_waves == 1
    check_fallback(g, 65536, 1, 1024)
    check_fallback(g, 65536, 2, 1024)
    for G in (4, 8, 16):
        shared(g, 65536, G, 1024)
    g4 = desc(B=4)
    check_fallback(g4, 65536, 4, 1024)
    g8 = desc(B=8)
    shared(g8, 65536, 8, 1024)
    # GQA with 16 heads per KV head (key streams at 16-63 rows): 2 requests
    # (32 rows) fall back, 8 (128 rows) share
    g16 = desc(B=16, Hq=32, Hkv=2)
    check_fallback(g16, 65536, 2, 1024)
    shared(g16, 65536, 8, 1024)
    # draft rows (4 positions x 8 heads = 32 rows at head dim 256: two row
    # tiles on a ring): groups of two (64 rows) share
    dr = desc(B=8, q_len=4, Hq=32, Hkv=4, Dk=256, Dv=256, causal=1)
    shared(dr, 2048, 2, 1024)
    check_fallback(dr, 2048, 1, 1024)
    # fp32 (vector ALUs), 4 heads per KV head: groups of 8 (32 rows) share,
    # groups of 4 (16 rows) fall back
    f = desc(B=16, Hq=4, Hkv=1, Dk=64, Dv=64, dtype=sk.ATTN_F32)
    shared(f, 4096, 8, 1024)
    check_fallback(f, 4096, 4, 1024)
    # validation comes first: a prefix too long for the context fails either way
    with pytest.raises(sk.AttnDecodeError):
        sk.attn_decode_plan_prefix(dr, 2048, 1, 2048)


@pytest.mark.parametrize("args,status", [
    ((7, 100), sk.ATTN_EINVAL),        # group does not divide the batch
    ((0, 100), sk.ATTN_EINVAL),
    ((8, -16), sk.ATTN_EINVAL),
    ((8, 100), sk.ATTN_EINVAL),        # not a whole number of 16-key pages
    ((8, 1 << 20), sk.ATTN_EINVAL),    # longer than the longest context
])
def test_prefix_plan_rejects(args, status):
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_plan_prefix(desc(B=16), 65536, *args)
    assert ei.value.status == status


def test_prefix_plan_flags_and_run_errors():
    d = desc(B=16, Hq=16, Hkv=1, Dk=576, Dv=512, P=1, maxp=68000, alias=1, pages=655360)
    for bad in (sk.ATTN_PLAN_FUSED_MERGE, sk.ATTN_PLAN_POLICY_P2, 32):
        with pytest.raises(sk.AttnDecodeError) as ei:
            sk.attn_decode_plan_prefix(d, 1000, 8, 600, bad)
        assert ei.value.status == sk.ATTN_EINVAL
    assert sk.attn_decode_plan_prefix(d, 1000, 8, 600, sk.ATTN_PLAN_NO_XCD_REMAP).shared.xcd_remap == 0
    # causal rows: every row must see the whole prefix
    dc = desc(B=4, q_len=4, Hq=32, Hkv=4, Dk=256, Dv=256, causal=1)
    sk.attn_decode_plan_prefix(dc, 2048, 2, 2032)   # 2032 + 4 - 1 <= 2048
    with pytest.raises(sk.AttnDecodeError):
        sk.attn_decode_plan_prefix(dc, 2048, 2, 2048)
    pp = sk.attn_decode_plan_prefix(d, 1000, 8, 600)
    fake = 1 << 20
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run_prefix(pp, fake, fake, fake, fake, fake, 0.1, fake, None, fake, 16, stream=0)
    assert ei.value.status == sk.ATTN_EWORKSPACE
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run_prefix(pp, None, fake, fake, fake, fake, 0.1, fake, None, fake, 1 << 30, stream=0)
    assert ei.value.status == sk.ATTN_EINVAL
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run_prefix(pp, fake, fake, fake, fake, fake, 0.1, None, None, fake, 1 << 30, stream=0)
    assert ei.value.status == sk.ATTN_EINVAL


def test_noalloc_rejects_plans_beyond_its_scratch_before_any_hip_call():
    """The no-allocation entry point checks the plan's workspace against its
    static scratch, and the plan flags, before it touches the HIP runtime."""
    fake = 1 << 20
    mla = desc(B=64, Hq=128, Hkv=1, Dk=576, Dv=512, P=1, maxp=16384, alias=1, pages=1 << 20)
    big = sk.attn_decode_plan(mla, 16384, 8, 0)           # 8 splits: 268 MB of partials
    assert sk.attn_decode_workspace_layout(big, 8)[2] > sk.NOALLOC_SCRATCH_BYTES
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run_noalloc(big, fake, fake, fake, fake, fake, 0.04, 8, fake, None, stream=0)
    assert ei.value.status == sk.ATTN_EWORKSPACE
    assert "static scratch" in sk.attn_decode_last_error()
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run_noalloc(big, fake, fake, fake, fake, fake, 0.04, 9, fake, None, stream=0)
    assert ei.value.status == sk.ATTN_EWORKSPACE             # beyond the plan's max_splits
    fused = sk.attn_decode_plan(mla, 16384, 2, sk.ATTN_PLAN_FUSED_MERGE)
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run_noalloc(fused, fake, fake, fake, fake, fake, 0.04, 2, fake, None, stream=0)
    assert ei.value.status == sk.ATTN_EUNSUPPORTED
    # every full-size workload's default plan fits the scratch
    from workloads import CONFIGS
    for w in CONFIGS.values():
        ks = (w.num_kv_heads * w.page_size * w.head_dim_qk, w.page_size * w.head_dim_qk, w.head_dim_qk)
        vs = ks if w.v_aliases_k else (w.num_kv_heads * w.page_size * w.head_dim_v, w.page_size * w.head_dim_v,
                                       w.head_dim_v)
        d = sk.make_desc(batch=w.batch, q_len=w.q_len, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                         head_dim_qk=w.head_dim_qk, head_dim_v=w.head_dim_v, page_size=w.page_size,
                         max_pages_per_req=w.max_pages_per_req,
                         dtype=sk.ATTN_F32 if w.kv_dtype == "f32" else sk.ATTN_BF16, causal=int(w.causal),
                         v_aliases_k=int(w.v_aliases_k), num_pages=w.pool_pages, k_strides=ks, v_strides=vs)
        p = sk.attn_decode_plan(d, max(w.context_lens), w.num_splits, 0)
        assert p.num_splits == 1 or p.workspace_bytes <= sk.NOALLOC_SCRATCH_BYTES, w.name


def test_xcd_order_only_for_batched_single_position_decode():
    """The split-major XCD-contiguous order is planned for decode batches
    (requests that may share KV on one XCD's L2), not for one request and not
    for several query positions per request."""
    assert sk.attn_decode_plan(mla_desc(48), 68000, 0).xcd_remap == 1
    assert sk.attn_decode_plan(desc(B=4, maxp=2048), 2048, 0).xcd_remap == 1
    assert sk.attn_decode_plan(desc(B=1), 65536, 0).xcd_remap == 0
    assert sk.attn_decode_plan(desc(B=4, q_len=4, causal=1, maxp=2048), 2048, 0).xcd_remap == 0
    assert sk.attn_decode_plan(mla_desc(48), 68000, 0, sk.ATTN_PLAN_NO_XCD_REMAP).xcd_remap == 0


def drafts_desc(B=6):
    return desc(B=B, q_len=4, Hq=32, Hkv=4, Dk=256, Dv=256, P=16, maxp=128, causal=1, pages=768)


def test_plan_lens_fixes_one_split_length_for_ragged_batches():
    """Known lengths: the policy gives every request the same split length
    (in proportion to its length, per-request split counts) when that
    shortens the longest walk and the live workgroups fit one round."""
    lens = [256, 512, 768, 1024, 1536, 2048]
    p = sk.attn_decode_plan_lens(drafts_desc(), lens, 0, 0)
    assert p.split_chunk == 128 and p.num_splits == 16 and p.max_splits == 16
    # the work list: one (request, split) item per 128 keys, request-major
    assert list(p.split_start[:7]) == [0, 2, 6, 12, 20, 32, 48] and p.live_splits == 48
    assert all(x == 0 for x in p.split_start[7:])
    assert p.live_splits * 4 * p.head_tiles == 192 <= 256
    # the split-count rule for the same batch walks 256 keys per split
    q = sk.attn_decode_plan(drafts_desc(), 2048, 0)
    assert q.split_chunk == 0 and q.num_splits == 8
    b, e = sk.attn_decode_split_range(q, 2048, 0, 0)
    assert e - b == 256
    assert p.key != q.key
    # every request's splits follow the oracle's fixed-length rule
    for L in list(range(0, 2049, 7)) + lens:
        ref = oracle.split_bounds(L, p.num_splits, 64, chunk=p.split_chunk)
        for s in range(p.num_splits):
            assert sk.attn_decode_split_range(p, L, 0, s) == ref[s], (L, s)


def test_plan_lens_on_equal_lengths_equals_plan():
    for d, lens in ((mla_desc(48), [68000] * 48), (desc(), [65536]), (desc(B=3, maxp=2048), [2048] * 3),
                    (desc(B=64, Hq=128, Hkv=1, Dk=576, Dv=512, P=1, maxp=16384, alias=1, pages=1 << 20),
                     [16384] * 64)):
        a = sk.attn_decode_plan_lens(d, lens, 0, 0).as_dict()
        b = sk.attn_decode_plan(d, max(lens), 0, 0).as_dict()
        assert a == b


def test_plan_lens_forced_and_p2_splits_keep_the_split_count_rule():
    lens = [256, 512, 768, 1024, 1536, 2048]
    for n, f in ((5, 0), (0, sk.ATTN_PLAN_POLICY_P2)):
        a = sk.attn_decode_plan_lens(drafts_desc(), lens, n, f)
        assert a.split_chunk == 0
        assert a.as_dict() == sk.attn_decode_plan(drafts_desc(), 2048, n, f).as_dict()


def test_fixed_split_length_plans_run_with_their_own_split_count():
    p = sk.attn_decode_plan_lens(drafts_desc(), [256, 512, 768, 1024, 1536, 2048], 0, 0)
    fake = 1 << 20
    for S in (1, 8, 15):
        with pytest.raises(sk.AttnDecodeError) as ei:
            sk.attn_decode_run(p, fake, fake, fake, fake, fake, 0.1, S, fake, None, fake, 1 << 30, stream=0)
        assert ei.value.status == sk.ATTN_EINVAL
        with pytest.raises(sk.AttnDecodeError) as ei:
            sk.attn_decode_split_range(p, 100, S, 0)
        assert ei.value.status == sk.ATTN_EINVAL
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_run(p, fake, fake, fake, fake, fake, 0.1, 17, fake, None, fake, 1 << 30, stream=0)
    assert ei.value.status == sk.ATTN_EWORKSPACE


def test_plan_lens_argument_errors():
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_plan_lens(drafts_desc(), [256, -1, 3, 4, 5, 6], 0, 0)
    assert ei.value.status == sk.ATTN_EINVAL
    with pytest.raises(sk.AttnDecodeError) as ei:
        sk.attn_decode_plan_lens(drafts_desc(), [256, 100000, 3, 4, 5, 6], 0, 0)   # beyond the page table
    assert ei.value.status == sk.ATTN_EINVAL
    L = sk.lib()
    st = L.attn_decode_plan_lens(ctypes.byref(drafts_desc()), None, 0, 0, ctypes.byref(sk.AttnDecodePlan()))
    assert st == sk.ATTN_EINVAL


def test_split_table_only_for_small_unfused_batches():
    """The work list lives in the plan (ATTN_MAX_SPLIT_TABLE requests) and
    the in-kernel merge counts a fixed number of splits per row group, so
    larger batches and fused plans keep the split-count rule."""
    lens = [256, 512, 768, 1024, 1536, 2048] * 11                 # 66 requests
    d = desc(B=66, q_len=4, Hq=32, Hkv=4, Dk=256, Dv=256, P=16, maxp=128, causal=1, pages=10000)
    p = sk.attn_decode_plan_lens(d, lens, 0, 0)
    assert p.split_chunk == 0 and p.live_splits == 0
    f = sk.attn_decode_plan_lens(drafts_desc(), [256, 512, 768, 1024, 1536, 2048], 0, sk.ATTN_PLAN_FUSED_MERGE)
    assert f.split_chunk == 0 and f.live_splits == 0
    # zero-length requests own no work item
    z = sk.attn_decode_plan_lens(drafts_desc(), [0, 512, 0, 1024, 1536, 2048], 0, 0)
    assert z.split_chunk > 0
    st = list(z.split_start[:7])
    assert st[1] - st[0] == 0 and st[3] - st[2] == 0 and z.live_splits == st[6]
