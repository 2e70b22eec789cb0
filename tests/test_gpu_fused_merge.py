"""GPU parity of the in-kernel merge (plans made with ATTN_PLAN_FUSED_MERGE):
the workgroup that writes a row group's last split merges the group inside
the stage-1 launch.  Same bar as the two-launch path against the CPU oracle
(bf16 1e-2 relative per row, log-sum-exp 1e-3 absolute); in addition the
partials equal the two-launch path's bit for bit (stage 1 is unchanged), the
counters are back at zero after every call, and split counts above 64 or of
one take the other paths of run() on the same plan.
"""

import numpy as np
import pytest

from tests.gpu_helpers import Decode, lse_err, row_rel_err, say, tol_for
from tests.test_gpu_parity import _RANDOM, check_against_oracle, inputs, small_cases
from workloads import generate, get

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import split_kv_paged_page_amd as sk  # noqa: E402

FUSED = sk.ATTN_PLAN_FUSED_MERGE

# bf16 cases: one and two head tiles, head dims 64-576, ragged and empty
# contexts, causal drafts and prefill rows (the fp32 plans have no fused form)
CASES = ["gqa_64k_s5000", "gqa_64k_b3_ragged", "mla_b48_b16", "mla_wide_b4", "varlen_drafts", "gqa_g4_bf16",
         "gqa_g20_bf16", "d256_g8", "mla_h4", "gqa_d64_bf16", "prefill_small_d64", "prefill_q20_d64",
         "prefill_q30_d128", "mla_h16_b1"]


def fused_splits(d_default: int) -> int:
    return min(max(d_default, 2), 64)


@pytest.mark.parametrize("name", CASES)
def test_fused_parity_small(name):
    w = small_cases()[name]
    inp = inputs(name, w)
    ref = Decode(inp)
    S = fused_splits(ref.S)
    if S != ref.S:      # the reference plan must hold S splits too
        ref = Decode(inp, num_splits=S)
    say(f"fused {name} S={S}: two-launch run")
    ref.run(S)
    d = Decode(inp, num_splits=S, flags=FUSED)
    assert (d.counters() == 0).all()
    say(f"fused {name} S={S}: fused run")
    d.run(S)
    e_out, e_lse = check_against_oracle(d, tol_for(w), S=S)
    assert (d.counters() == 0).all()
    # stage 1 is the same kernel: the partials carry the same bits
    assert np.array_equal(d.used_ws_bits(S), ref.used_ws_bits(S))
    # the two merges differ only in rounding order
    assert row_rel_err(d.out_f64(), ref.out_f64()) <= 1e-2
    assert lse_err(d.lse_f64(), ref.lse_f64()) <= 1e-5
    print(f"{name}: S={S} tiles={d.plan.head_tiles} out {e_out:.2e} lse {e_lse:.2e}")


def test_fused_repeated_calls_and_split_changes():
    # Every call leaves the counters at zero, so calls with other split
    # counts follow on the same workspace; S = 1 (direct output) and S > 64
    # (two launches) leave the counters alone.
    w = small_cases()["gqa_g20_bf16"]
    inp = inputs("gqa_g20_bf16", w)
    d = Decode(inp, flags=FUSED, max_splits=100)
    for S in (64, 5, 2, 64, 17, 1, 100, 3):
        say(f"fused repeat S={S}")
        d.run(S)
        check_against_oracle(d, tol_for(w), S=S, check_splits=S > 1)
        assert (d.counters() == 0).all(), S


def test_fused_output_without_lse():
    w = small_cases()["varlen_drafts"]
    inp = inputs("varlen_drafts", w)
    d = Decode(inp, flags=FUSED)
    say("fused without lse")
    d.poison()
    t = d.t
    sk.attn_decode_run(d.plan, t["q"], t["k_cache"], d.v, t["page_table"], t["context_lens"], float(inp.scale),
                       d.S, d.out, None, d.ws)
    torch.cuda.synchronize()
    assert torch.isnan(d.lse).all()          # untouched
    d.lse.copy_(Decode(inp).run().lse)
    check_against_oracle(d, tol_for(w), check_splits=False)
    assert (d.counters() == 0).all()


@pytest.mark.parametrize("name", ["mla_b48_b16", "varlen_drafts", "prefill_q20_d64"])
def test_fused_graph_replays_match_eager(name):
    w = small_cases()[name]
    inp = inputs(name, w)
    d = Decode(inp, flags=FUSED)
    S = fused_splits(d.S)
    say(f"fused graph {name} eager S={S}")
    d.run(S)
    e_out, e_lse, e_ws = d.out.clone(), d.lse.clone(), d.used_ws_bits(S)
    t = d.t
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    d.poison()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        sk.attn_decode_run(d.plan, t["q"], t["k_cache"], d.v, t["page_table"], t["context_lens"],
                           float(inp.scale), S, d.out, d.lse, d.ws, stream=s.cuda_stream)
    for r in range(3):
        d.poison()
        torch.cuda.synchronize()
        say(f"fused graph {name} replay {r}")
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out.view(torch.int16), e_out.view(torch.int16)), r
        assert torch.equal(d.lse.view(torch.int32), e_lse.view(torch.int32)), r
        assert np.array_equal(d.used_ws_bits(S), e_ws), r
        assert (d.counters() == 0).all(), r


@pytest.mark.parametrize("name,S,requests,lens", [("varlen_drafts", None, None, False),
                                                  ("varlen_drafts", None, None, True),
                                                  ("mla_b48", None, (0, 13, 47), False),
                                                  ("mla_wide", None, (0, 63), False), ("gqa_64k", 64, None, False),
                                                  ("prefill_varlen_d64", 8, None, False)])
def test_fused_full_size_sampled(name, S, requests, lens):
    # lens: planned with the batch's lengths; a fused plan keeps the
    # split-count rule (its counters expect the same split count per row group)
    w = get(name)
    say(f"fused full-size {name} lens={lens}: generating inputs")
    inp = generate(w)
    d = Decode(inp, num_splits=S or 0, flags=FUSED, lens=lens)
    assert d.chunk is None and d.plan.live_splits == 0
    assert 2 <= d.S <= 64, d.S
    say(f"fused full-size {name}: run S={d.S}")
    d.run()
    e_out, e_lse = check_against_oracle(d, tol_for(w), requests=requests)
    assert (d.counters() == 0).all()
    if requests is not None:
        assert not torch.isnan(d.out).any() and torch.isfinite(d.lse).all()
    print(f"{name}: S={d.S} out {e_out:.2e} lse {e_lse:.2e}")


_RANDOM_BF16 = [k for k, w in _RANDOM.items() if w.kv_dtype == "bf16"]


@pytest.mark.parametrize("name", _RANDOM_BF16)
def test_fused_parity_random_shapes(name):
    # the bf16 shapes of the two-launch random sweep (head dims 64-576, groups
    # 1-40, causal rows, page sizes 1-64, empty and short contexts), each at
    # its split count clamped to the fused range 2-64
    w = _RANDOM[name]
    inp = generate(w)
    probe = Decode(inp, num_splits=w.num_splits)
    S = fused_splits(probe.S)
    say(f"fused random {name}: B={w.batch} q_len={w.q_len} heads={w.num_q_heads}/{w.num_kv_heads} "
        f"dims={w.head_dim_qk}/{w.head_dim_v} P={w.page_size} causal={w.causal} ctx={w.context_lens} S={S}")
    d = Decode(inp, num_splits=S, flags=FUSED).run()
    e_out, e_lse = check_against_oracle(d, tol_for(w), S=S)
    assert (d.counters() == 0).all()
    print(f"{name}: S={S} rows/wg={d.plan.rows_per_wg} out {e_out:.2e} lse {e_lse:.2e}")
