"""The benchmark's algorithmic work (bytes and flops per launch), restated
from the oracle's visible-key rule and the workload shapes (no GPU)."""

import pytest

import bench
import oracle
from workloads import CONFIGS


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_flops_count_every_visible_key(name):
    w = CONFIGS[name]
    pairs = sum(oracle.visible_keys(int(L), w.q_len, j, w.causal)
                for L in w.context_lens for j in range(w.q_len))
    assert bench.algorithmic_flops(w) == 2 * pairs * w.num_q_heads * (w.head_dim_qk + w.head_dim_v)


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_bytes_count_each_kv_row_once(name):
    w = CONFIGS[name]
    es = 4 if w.kv_dtype == "f32" else 2
    row = w.head_dim_qk * es + (0 if w.v_aliases_k else w.head_dim_v * es)
    kv, total = bench.algorithmic_bytes(w, 4)
    assert kv == sum(w.context_lens) * w.num_kv_heads * row
    rows = w.batch * w.q_len * w.num_q_heads
    assert total > kv + rows * 4 * (w.head_dim_v + 1) * 4 - 1      # partials of 4 splits included
    _, one = bench.algorithmic_bytes(w, 1)
    assert one < total                                               # one split: the output instead


def test_bytes_count_only_the_work_lists_partials():
    w = CONFIGS["varlen_drafts"]
    counts = [2, 4, 6, 8, 12, 16]           # 128-key splits of the drafts' lengths
    kv, dense = bench.algorithmic_bytes(w, 16)
    _, listed = bench.algorithmic_bytes(w, 16, counts)
    per_split_row = w.q_len * w.num_q_heads * (w.head_dim_v + 1) * 4
    assert dense - listed == (16 * w.batch - sum(counts)) * per_split_row
