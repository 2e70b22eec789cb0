"""Benchmark: split-KV paged decode on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config gqa_64k] [--splits S]

One step = one decode op (stage 1 + stage 2) over one batch of the workload.
Inputs are seeded synthetic data resident in HBM before timing starts.  The
KV pool is replicated R times and step i reads replica i mod R, so every step
reads KV that no cache still holds (R x touched bytes >= 1 GiB, four times the
last-level cache).  The K timed steps run as one captured HIP graph
(launch overhead excluded) bracketed by torch.cuda.synchronize(); HIP events
on the launch stream give the time.  The graph is replayed five times and
the median replay is reported (every replay's figure is in the line).  Stage
1 alone is timed the same way (a graph of K stage-1 launches) for the
roofline entry.

Prints one JSON line.  value = logical KV bytes per op / time per op (GB/s)
of the headline workload (--config, 64K GQA by default).  The default run
also times the other decode workloads (--extra): the tiny fp32 check, MLA
batch 48 with and without shared prefixes, one MLA request, the 128-head MLA,
the varlen drafts and 8 GQA requests sharing a 61,440-key prefix, each under
"configs" with its whole-op and stage-1 times, its own
stage-1 roofline entry, a plain cold read of the same KV bytes (unique bytes
where prefixes are shared) and, for shared prefixes, the unique-bytes rate.
A name ending in "+prefix" is that workload again through the shared-prefix
plan (attn_decode_plan_prefix: each group's shared keys scored once for all
its members' rows), whole op only; --prefix times only that for --config.

Beside stage 1 the line carries a plain device-memory read timed the same
way (libsplitkv_probe.so): a 2 GiB streaming read, the part's practical read
rate, and cold reads of exactly the workload's KV byte count, which pay the
same launch, start-up and tail costs as stage 1 with no page walk and no
arithmetic.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# MI355X dense peaks: bf16 matrix cores (the bf16 kernel's Q.K and P.V), fp32
# vector ALUs (the fp32 kernel).
MFMA_BF16_PEAK_TFLOPS = 2500.0
VALU_F32_PEAK_TFLOPS = 157.3
PROBE_GRIDS = (1024, 2048, 4096)   # read-probe workgroup counts tried (256 lanes each); the fastest is used


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="gqa_64k")
    ap.add_argument("--extra", default=EXTRA_CONFIGS,
                    help="comma-separated workloads timed after the headline one, each reported under "
                         "'configs' ('' for none)")
    ap.add_argument("--splits", type=int, default=0, help="force the split count (0: planner policy)")
    ap.add_argument("--batch", type=int, default=0,
                    help="the workload with B requests of its first request's length (the aiter PR's "
                         "concurrency sweep; 0: as named)")
    ap.add_argument("--flags", type=int, default=0, help="attn_decode_plan flags")
    ap.add_argument("--replicas", type=int, default=0, help="KV pool copies to rotate (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true", help="skip the plain device-memory read beside stage 1")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step eagerly instead of from a captured graph (counter runs)")
    ap.add_argument("--prefix", action="store_true",
                    help="time the workload through the shared-prefix plan (whole op only)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 20 device-to-device copies of MIB MiB (HBM counter calibration)")
    return ap.parse_args()


def algorithmic_bytes(w, S, split_counts=None):
    """Bytes one stage-1 launch must move at minimum: every visible key of
    every KV head once (V counted once when it aliases K), the page-table
    entries, q, and the partial outputs + log-sum-exps it writes (with one
    split: the output and log-sum-exp themselves; with a work list,
    split_counts[b] partials per row of request b)."""
    es = w.elem_bytes
    kv = w.logical_kv_bytes()
    pt = sum(-(-c // w.page_size) for c in w.context_lens) * 4
    # q of the rows that see at least one key (causal rows before a short
    # sequence's first token see none)
    seen = sum(min(w.q_len, L) if w.causal else (w.q_len if L > 0 else 0) for L in w.context_lens)
    q = seen * w.num_q_heads * w.head_dim_qk * es
    rows = w.batch * w.q_len * w.num_q_heads
    if S == 1:
        part = rows * (w.head_dim_v * es + 4)
    elif split_counts is not None:
        part = sum(split_counts) * w.q_len * w.num_q_heads * (w.head_dim_v + 1) * 4
    else:
        part = rows * S * (w.head_dim_v + 1) * 4
    return kv, kv + pt + q + part


def algorithmic_flops(w):
    """2 x the multiply-adds the method needs: every query row against every
    key it may see, over Dk for Q.K and Dv for P.V (causal rows see
    max(0, L - q_len + 1 + j) keys)."""
    pairs = 0
    for L in w.context_lens:
        if w.causal:
            first = L - w.q_len + 1
            pairs += sum(max(0, first + j) for j in range(w.q_len))
        else:
            pairs += w.q_len * L
    return 2 * pairs * w.num_q_heads * (w.head_dim_qk + w.head_dim_v)


def time_eager(fn_steps, steps, stream):
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    with torch.cuda.stream(stream):
        for i in range(steps):
            fn_steps(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    return ms, None, [ms]


def copy_probe(mib):
    """A plain copy kernel of known size, for scaling HBM byte counters."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(20):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 20}), flush=True)


WARM_SECONDS = 0.3   # untimed replays before the timed ones: the part's clocks ramp up over this


def time_graph(fn_steps, steps, stream, rounds=5):
    """Capture fn_steps(i) for i < steps into one graph; replay it untimed
    for WARM_SECONDS (graph upload, first touches, and the clock ramp: on
    the compute-heavier configs successive replays ran up to 10% faster
    over the first few hundred milliseconds), then `rounds` times, each
    between HIP events; return (median ms per replay, graph, every replay's
    ms)."""
    import statistics

    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            fn_steps(i)
    torch.cuda.synchronize()
    times = []
    with torch.cuda.stream(stream):     # replay() launches on the current stream
        t0 = time.perf_counter()
        while True:                     # untimed replays
            g.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= WARM_SECONDS:
                break
        for _ in range(rounds):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
    return statistics.median(times), g, times


def read_probe_line(kv_bytes, steps, stream):
    """Plain device-memory reads timed like stage 1 (graph replays, median of
    five): a 2 GiB streaming read at each grid of PROBE_GRIDS, then, at the
    fastest grid, `steps` cold reads of kv_bytes each, rotating over copies
    that together exceed 1 GiB."""
    import torch
    from split_kv_paged_page_amd.read_probe import read_probe
    sink = torch.zeros(max(PROBE_GRIDS), dtype=torch.int32, device="cuda")
    sid = stream.cuda_stream
    big_n = 1 << 31
    big = torch.empty(big_n // 4, dtype=torch.int32, device="cuda")
    big_gbs = {}
    for wgs in PROBE_GRIDS:
        ms, g, _ = time_graph(lambda i: read_probe(big.data_ptr(), big_n, wgs, sink.data_ptr(), sid), 4, stream)
        del g
        big_gbs[wgs] = big_n * 4 / (ms * 1e-3) / 1e9
    del big
    wgs = max(big_gbs, key=big_gbs.get)
    n = -(-kv_bytes // 256) * 256
    R = max(1, -(-(1 << 30) // n))
    pool = torch.empty(R * n // 4, dtype=torch.int32, device="cuda")
    base = pool.data_ptr()
    ms, g, _ = time_graph(lambda i: read_probe(base + (i % R) * n, n, wgs, sink.data_ptr(), sid), steps, stream)
    del g, pool
    same_us = ms * 1e3 / steps
    return {"kernel": "plain read: each workgroup one contiguous share, 16 B per lane, 8 loads in flight",
            "workgroups": wgs, "large_read_bytes": big_n, "large_read_gbs": round(big_gbs[wgs], 1),
            "large_read_gbs_by_grid": {str(k): round(v, 1) for k, v in big_gbs.items()},
            "same_bytes": n, "same_bytes_copies": R, "same_bytes_cold_us": round(same_us, 3),
            "same_bytes_gbs": round(n / (same_us * 1e-6) / 1e9, 1)}


def read_probe_same_bytes(nbytes, steps, stream, wgs):
    """Cold plain reads of nbytes each (graph replays, median of five),
    rotating over copies that together exceed 1 GiB."""
    import torch
    from split_kv_paged_page_amd.read_probe import read_probe
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    n = -(-nbytes // 256) * 256
    R = max(1, -(-(1 << 30) // n))
    pool = torch.empty(R * n // 4, dtype=torch.int32, device="cuda")
    base = pool.data_ptr()
    ms, g, _ = time_graph(lambda i: read_probe(base + (i % R) * n, n, wgs, sink.data_ptr(), stream.cuda_stream),
                          steps, stream)
    del g, pool
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    us = ms * 1e3 / steps
    return {"same_bytes": n, "same_bytes_copies": R, "workgroups": wgs, "same_bytes_cold_us": round(us, 3),
            "same_bytes_gbs": round(n / (us * 1e-6) / 1e9, 1)}


def cpu_baseline(inp, kv_bytes, budget_s):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.decode_reference(inp)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 50:
            break
    med = float(np.median(times))
    return {"value": kv_bytes / med / 1e9, "unit": "GB/s (logical KV bytes / oracle time per op)",
            "cores": int(threads), "kind": "oracle",
            "sample": f"whole decode op of the same workload, float64 NumPy oracle, {len(times)} runs, "
                      f"median {med * 1e3:.1f} ms/op, host os.cpu_count()={os.cpu_count()}"}


# Configurations timed beside the headline one in the default run, each with
# its own stage-1 roofline: the tiny fp32 check, MLA batch 48 with and
# without shared prefixes, the 128-head MLA and the varlen drafts.
EXTRA_CONFIGS = "gqa_tiny_f32,mla_b48,mla_b48+prefix,mla_b48_ctl,mla_b1,mla_wide,varlen_drafts,gqa_64k_b8_shared,gqa_64k_b8_shared+prefix"
PREFIX_SUFFIX = "+prefix"   # an --extra entry <workload>+prefix: that workload through the shared-prefix plan


def measure(w, args, stream, splits=0, flags=0, want_inputs=False):
    """Plan, upload and time one workload: the whole op and stage 1 alone,
    each as graph replays over cold KV.  Returns (summary dict, inputs or
    None); every device buffer is released before returning."""
    import torch

    import split_kv_paged_page_amd as sk
    from workloads import generate
    from workloads.torch_io import upload

    inp = generate(w)
    t = upload(inp, "cuda")
    desc = sk.make_desc_from_tensors(t["q"], t["k_cache"], t["v_cache"], t["page_table"],
                                     head_dim_v=w.head_dim_v, causal=w.causal)
    # the workload's lengths are known on the host (ragged batches may get
    # one fixed split length for every request)
    # a workload without shared prefixes shares no page between requests,
    # which the plan may be told
    if not w.prefix_group:
        flags |= sk.ATTN_PLAN_PRIVATE_PAGES
    plan = sk.attn_decode_plan_lens(desc, [int(x) for x in w.context_lens], splits or w.num_splits, flags)
    S = plan.num_splits
    counts = None
    if plan.live_splits > 0:   # work list: request b writes its own split count's partials
        counts = [plan.split_start[b + 1] - plan.split_start[b] for b in range(w.batch)]
    kv_bytes, alg_bytes = algorithmic_bytes(w, S, counts)
    touched = w.unique_kv_bytes()
    R = args.replicas or max(1, -(-(1 << 30) // touched))
    ks = [t["k_cache"]] + [t["k_cache"].clone() for _ in range(R - 1)]
    vs = [t["v_cache"]] + [t["v_cache"].clone() for _ in range(R - 1)] if t["v_cache"] is not None else ks
    dt = torch.float32 if w.kv_dtype == "f32" else torch.bfloat16
    out = torch.empty((w.batch, w.q_len, w.num_q_heads, w.head_dim_v), dtype=dt, device="cuda")
    lse = torch.empty((w.batch, w.q_len, w.num_q_heads), dtype=torch.float32, device="cuda")
    ws = torch.empty(plan.workspace_bytes // 4, dtype=torch.float32, device="cuda")
    scale = float(inp.scale)
    # the in-kernel merge's counters start at zero (a no-op for other plans)
    sk.attn_decode_workspace_init(plan, ws, stream=stream.cuda_stream)

    def step(i):
        r = i % R
        sk.attn_decode_run(plan, t["q"], ks[r], vs[r], t["page_table"], t["context_lens"], scale, S,
                           out, lse, ws, stream=stream.cuda_stream)

    def stage1(i):
        r = i % R
        if S == 1:
            # one split: the op is stage 1 alone, writing the output itself
            # (the partials call would write fp32 partials instead)
            step(i)
            return
        sk.attn_decode_partials(plan, t["q"], ks[r], vs[r], t["page_table"], t["context_lens"], scale, S,
                                ws, stream=stream.cuda_stream)

    # warmup (eager)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    timer = time_eager if args.eager else time_graph
    ms, g, op_rounds = timer(step, args.steps, stream)
    del g
    ms1, g1, s1_rounds = timer(stage1, args.steps, stream)
    del g1
    del ks, vs, t, out, lse, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    us_op = ms * 1e3 / args.steps
    us_s1 = ms1 * 1e3 / args.steps
    kv_gbs = kv_bytes / (us_op * 1e-6) / 1e9
    ach = alg_bytes / (us_s1 * 1e-6) / 1e9
    flops = algorithmic_flops(w)
    peak_tf = MFMA_BF16_PEAK_TFLOPS if w.kv_dtype == "bf16" else VALU_F32_PEAK_TFLOPS
    # the kernel is bound by whichever of HBM and the compute units needs longer
    compute_bound = flops / (peak_tf * 1e12) > alg_bytes / (HBM_PEAK_GBS * 1e9)

    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"stage1_traffic_{w.name}.json")
    if os.path.exists(tfile) and not args.eager:
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("plan_key") == str(plan.key) and tr.get("kernel_source_hash") == source_hash():
            traffic = tr.get("bytes_per_launch")

    res = {
        "workload": w.name,
        "us_per_op": round(us_op, 3),
        "stage1_us": round(us_s1, 3),
        "kv_gbs": round(kv_gbs, 1),
        "kv_hbm_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "us_per_op_rounds": [round(x * 1e3 / args.steps, 3) for x in op_rounds],
        "stage1_us_rounds": [round(x * 1e3 / args.steps, 3) for x in s1_rounds],
        "tflops_per_s": round(flops / (us_op * 1e-6) / 1e12, 2),
        "num_splits": S, "split_chunk": plan.split_chunk, "rows_per_wg": plan.rows_per_wg,
        "head_tiles": plan.head_tiles,
        "stage1_waves": plan.stage1_waves, "xcd_remap": plan.xcd_remap, "plan_flags": plan.flags,
        "replicas": R, "kv_bytes_per_op": kv_bytes, "plan_key": str(plan.key),
        "roofline": {"bound": "hbm", "kernel": "stage1", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": alg_bytes, "alg_flops_per_launch": flops,
                     "launch_us": round(us_s1, 3)},
    }
    if compute_bound:
        tf = flops / (us_s1 * 1e-6) / 1e12
        res["roofline"].update({"bound": "mfma" if w.kv_dtype == "bf16" else "alu", "achieved": round(tf, 2),
                                "peak": peak_tf, "unit": "TFLOP/s", "frac": round(tf / peak_tf, 4),
                                "hbm_gbs": round(ach, 1)})
    if touched != kv_bytes:
        # shared prefixes: the logical rate counts every request's prefix
        # read (the re-reads come from cache); the unique bytes are what HBM
        # must deliver at least once
        res["unique_kv_bytes_per_op"] = touched
        res["stage1_unique_kv_gbs"] = round(touched / (us_s1 * 1e-6) / 1e9, 1)
        res["stage1_unique_kv_frac"] = round(touched / (us_s1 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    return res, (inp if want_inputs else None)


def measure_prefix(w, args, stream):
    """The workload through the shared-prefix plan (its groups of
    w.prefix_group requests share their first w.prefix_len keys): the whole op
    (shared pass, own pass, merge) as graph replays over cold KV."""
    import torch

    import split_kv_paged_page_amd as sk
    from workloads import generate
    from workloads.torch_io import upload

    inp = generate(w)
    t = upload(inp, "cuda")
    desc = sk.make_desc_from_tensors(t["q"], t["k_cache"], t["v_cache"], t["page_table"],
                                     head_dim_v=w.head_dim_v, causal=w.causal)
    # a batch that is not a whole number of groups (the sweep's B < 8) forms
    # groups of gcd(B, G) requests, which all share the prefix
    import math
    G = math.gcd(w.batch, w.prefix_group)
    plan = sk.attn_decode_plan_prefix(desc, int(max(w.context_lens)), G, w.prefix_len)
    kv_bytes, touched = w.logical_kv_bytes(), w.unique_kv_bytes()
    R = args.replicas or max(1, -(-(1 << 30) // touched))
    ks = [t["k_cache"]] + [t["k_cache"].clone() for _ in range(R - 1)]
    vs = [t["v_cache"]] + [t["v_cache"].clone() for _ in range(R - 1)] if t["v_cache"] is not None else ks
    dt = torch.float32 if w.kv_dtype == "f32" else torch.bfloat16
    out = torch.empty((w.batch, w.q_len, w.num_q_heads, w.head_dim_v), dtype=dt, device="cuda")
    lse = torch.empty((w.batch, w.q_len, w.num_q_heads), dtype=torch.float32, device="cuda")
    ws = torch.empty(plan.workspace_bytes // 4, dtype=torch.float32, device="cuda")
    scale = float(inp.scale)

    def step(i):
        r = i % R
        sk.attn_decode_run_prefix(plan, t["q"], ks[r], vs[r], t["page_table"], t["context_lens"], scale,
                                  out, lse, ws, stream=stream.cuda_stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    timer = time_eager if args.eager else time_graph
    ms, g, op_rounds = timer(step, args.steps, stream)
    del g, ks, vs, t, out, lse, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    us_op = ms * 1e3 / args.steps
    kv_gbs = kv_bytes / (us_op * 1e-6) / 1e9
    return {
        "workload": w.name, "plan": "shared prefix (attn_decode_plan_prefix)",
        "us_per_op": round(us_op, 3),
        "us_per_op_rounds": [round(x * 1e3 / args.steps, 3) for x in op_rounds],
        "kv_gbs": round(kv_gbs, 1), "kv_hbm_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "unique_kv_bytes_per_op": touched,
        "unique_kv_gbs": round(touched / (us_op * 1e-6) / 1e9, 1),
        "unique_kv_frac": round(touched / (us_op * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "tflops_per_s": round(algorithmic_flops(w) / (us_op * 1e-6) / 1e12, 2),
        "prefix_group": G, "prefix_len": w.prefix_len,
        # below the planner's row threshold the plan is the default one (no shared pass)
        "shared_pass": plan.prefix_len > 0,
        "shared_splits": plan.shared.num_splits if plan.prefix_len else 0, "own_splits": plan.own.num_splits,
        "shared_rows_per_wg": plan.shared.rows_per_wg, "shared_head_tiles": plan.shared.head_tiles,
        "own_rows_per_wg": plan.own.rows_per_wg, "replicas": R, "kv_bytes_per_op": kv_bytes,
        "plan_key": str(plan.key),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); the decode path does not "
              "shard across GPUs here", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    from workloads import get

    stream = torch.cuda.Stream()
    w = batch_workload(args.config, args.batch) if args.batch else get(args.config)
    if args.prefix:   # only the shared-prefix plan's op time, one JSON object
        if not w.prefix_group:
            print(f"bench.py: {w.name} has no shared prefixes", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(measure_prefix(w, args, stream)), flush=True)
        return
    head, inp = measure(w, args, stream, args.splits, args.flags, want_inputs=not args.no_cpu_baseline)
    kv_bytes = head["kv_bytes_per_op"]
    us_op, us_s1 = head["us_per_op"], head["stage1_us"]

    res = {
        "metric": "split-KV decode: µs per decode op and KV GB/s as % of MI355X HBM peak",
        "value": head["kv_gbs"],
        "unit": "GB/s (logical KV bytes per decode op / whole-op time)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us_op / 1e3, 6),
        "us_per_op": us_op,
        "kv_hbm_frac": head["kv_hbm_frac"],
        "stage1_us": us_s1,
        "rounds": len(head["us_per_op_rounds"]),
        "us_per_op_rounds": head["us_per_op_rounds"],
        "stage1_us_rounds": head["stage1_us_rounds"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "f32",
        "accumulate": "f32",
        "data": "synthetic (seeded N(0,1) values, seeded page tables; no dataset)",
        "config": {"workload": w.name, "batch": w.batch, "q_len": w.q_len, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim_qk": w.head_dim_qk, "head_dim_v": w.head_dim_v,
                   "page_size": w.page_size, "context": (w.context_lens[0] if len(set(w.context_lens)) == 1
                                                        else list(w.context_lens)),
                   "num_splits": head["num_splits"], "split_chunk": head["split_chunk"],
                   "rows_per_wg": head["rows_per_wg"],
                   "head_tiles": head["head_tiles"], "stage1_waves": head["stage1_waves"],
                   "xcd_remap": head["xcd_remap"], "plan_flags": head["plan_flags"], "replicas": head["replicas"],
                   "plan_key": head["plan_key"],
                   "kv_bytes_per_op": kv_bytes, "parallelism": "single GPU"},
        "tflops_per_s": head["tflops_per_s"],
        "roofline": head["roofline"],
    }
    if not args.no_read_probe:
        ach = head["roofline"]["alg_bytes_per_launch"] / (us_s1 * 1e-6) / 1e9
        rp = read_probe_line(kv_bytes, args.steps, stream)
        # stage 1 against a bare read: its time relative to a cold read of
        # the same KV bytes, and its rate relative to the streaming read
        rp["same_bytes_us_over_stage1_us"] = round(rp["same_bytes_cold_us"] / us_s1, 4)
        rp["stage1_gbs_over_large_read_gbs"] = round(ach / rp["large_read_gbs"], 4)
        res["read_probe"] = rp
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, kv_bytes, args.cpu_seconds)
    del inp
    extra = [n for n in args.extra.split(",") if n and n != w.name] if args.extra else []
    if extra:
        res["configs"] = {}
        for name in extra:
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            if name.endswith(PREFIX_SUFFIX):   # the named workload through the shared-prefix plan
                res["configs"][name] = measure_prefix(get(name[:-len(PREFIX_SUFFIX)]), args, stream)
                continue
            r, _ = measure(get(name), args, stream)
            if not args.no_read_probe:
                # a plain cold read of the same KV bytes (unique bytes where
                # prefixes are shared), timed the same way
                same = read_probe_same_bytes(r.get("unique_kv_bytes_per_op", r["kv_bytes_per_op"]),
                                             args.steps, stream, res.get("read_probe", {}).get("workgroups", 4096))
                same["same_bytes_us_over_stage1_us"] = round(same["same_bytes_cold_us"] / r["stage1_us"], 4)
                r["read_probe"] = same
            res["configs"][name] = r
    print(json.dumps(res), flush=True)


def batch_workload(name: str, batch: int):
    """The named workload with `batch` requests of its first request's
    length (the same page size, heads and sharing pattern), its page pool
    scaled in proportion and never below the pages the tables take."""
    from workloads import get, scaled
    w = get(name)
    w = scaled(name, batch=batch, pool_pages=-(-w.pool_pages * batch // w.batch))
    return scaled(name, batch=batch, pool_pages=max(w.pool_pages, w.pages_needed()))


def source_hash() -> str:
    """Hash of the library's sources without their // comments and blank
    lines (the sources hold no block comments and no "//" inside strings),
    so that counters taken on a build stay matched to it across comment
    edits."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "split_kv_paged_page_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            code = [ln.split("//", 1)[0].rstrip() for ln in fh]
        h.update(f.encode() + "\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
