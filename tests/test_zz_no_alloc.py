"""The no-allocation entry point on the GPU, through the C ABI:
attn_decode_run_noalloc (workspace in the library's static device scratch)
against attn_decode_run (caller workspace) on the same inputs.  Both run
the same kernels in the same order, so the outputs and log-sum-exps must be
bit-identical; they are also held to the oracle's tolerance.  Two calls in
a row, the second with a smaller input, check that nothing the first call
left in the shared scratch reaches the second one's output."""

import numpy as np
import pytest

import oracle
import split_kv_paged_page_amd as sk
from tests.gpu_helpers import Decode, lse_err, row_rel_err, say, tol_for
from workloads import generate, scaled

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _pairs():
    # (larger input, smaller input) per kernel family: bf16 GQA on the lone
    # matrix-core wave, MLA with four key streams, causal drafts on the
    # shared-tile ring, fp32 on the vector ALUs
    return {
        "gqa_bf16": (scaled("gqa_64k", context_lens=(5000, 777, 4100), pool_pages=1024, seed=61),
                     scaled("gqa_64k", context_lens=(300,), pool_pages=64, seed=62)),
        "mla": (scaled("mla_b48", batch=8, context_lens=(3000,) * 8, prefix_len=2000, seed=63),
                scaled("mla_b48", context_lens=(65, 1000), prefix_len=0, prefix_group=0, seed=64)),
        "drafts": (scaled("varlen_drafts", seed=65),
                   scaled("varlen_drafts", context_lens=(256, 515), seed=66)),
        "fp32": (scaled("gqa_64k", context_lens=(3000, 1, 777), kv_dtype="f32", seed=67),
                 scaled("gqa_64k", context_lens=(129,), kv_dtype="f32", pool_pages=32, seed=68)),
    }


def _noalloc(d: Decode, out, lse):
    t = d.t
    sk.attn_decode_run_noalloc(d.plan, t["q"], t["k_cache"], d.v, t["page_table"], t["context_lens"],
                               float(d.inp.scale), d.S, out, lse)


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


@pytest.mark.parametrize("name", list(_pairs()))
def test_noalloc_matches_run_on_two_calls(name):
    big, small = _pairs()[name]
    for tag, w in (("first (larger)", big), ("second (smaller)", small)):
        inp = generate(w)
        say(f"noalloc {name} {tag}: B={w.batch} ctx={w.context_lens} reference run")
        d = Decode(inp).run()
        ref_out, ref_lse = d.out.clone(), d.lse.clone()
        assert d.plan.workspace_bytes <= sk.NOALLOC_SCRATCH_BYTES
        out = torch.full_like(d.out, float("nan"))
        lse = torch.full_like(d.lse, float("nan"))
        say(f"noalloc {name} {tag}: S={d.S} no-allocation run")
        _noalloc(d, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref_out)), tag
        assert torch.equal(_bits(lse), _bits(ref_lse)), tag
        ro, rl = oracle.decode_reference(inp)
        assert row_rel_err(out.to(torch.float64).cpu().numpy(), ro) <= tol_for(w)
        assert lse_err(lse.double().cpu().numpy(), rl) <= 1e-3


def test_noalloc_forced_splits_and_graph_replay():
    """Split counts up to the scratch's reach in turn, then the call captured
    in a graph (after an eager call has looked the scratch up) and replayed
    with eager work between replays."""
    w = scaled("gqa_64k", context_lens=(20000, 3000), pool_pages=2048, seed=69)
    inp = generate(w)
    d = Decode(inp, max_splits=300)
    out = torch.empty_like(d.out)
    lse = torch.empty_like(d.lse)
    for S in (300, 7, 1, 64):
        d.S = S
        say(f"noalloc forced S={S}")
        d.run(S)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        _noalloc(d, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(d.out)), S
        assert torch.equal(_bits(lse), _bits(d.lse)), S
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    t = d.t
    say("noalloc graph capture S=64")
    with torch.cuda.graph(g, stream=s):
        sk.attn_decode_run_noalloc(d.plan, t["q"], t["k_cache"], d.v, t["page_table"], t["context_lens"],
                                   float(inp.scale), 64, out, lse, stream=s.cuda_stream)
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"noalloc graph replay {r}")
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(d.out)), r
        assert torch.equal(_bits(lse), _bits(d.lse)), r
