"""Seeded workload construction (no GPU): the page tables each workload
builds, the pages they take, and the bench's batch scaling."""

import numpy as np
import pytest

import bench
from workloads import CONFIGS
from workloads.gen import page_table_for


def _tables(w):
    perm = np.random.default_rng(w.seed).permutation(w.pool_pages).astype(np.int32)
    return page_table_for(w, perm)


def _used(w, pt):
    return [pt[b, :-(-int(L) // w.page_size)] for b, L in enumerate(w.context_lens)]


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_tables_take_the_pages_they_need(name):
    w = CONFIGS[name]
    used = _used(w, _tables(w))
    ids = np.concatenate(used) if used else np.zeros(0, np.int32)
    assert ids.size == 0 or (ids.min() >= 0 and ids.max() < w.pool_pages)
    assert len(np.unique(ids)) == w.pages_needed() <= w.pool_pages
    if not w.prefix_group:           # private pages: no page appears twice
        assert len(np.unique(ids)) == ids.size


def test_shared_prefixes_only_within_a_group():
    w = CONFIGS["mla_b48"]
    used = _used(w, _tables(w))
    npp = w.prefix_len // w.page_size
    for b in range(w.batch):
        g = b // w.prefix_group
        lead = used[g * w.prefix_group]
        assert np.array_equal(used[b][:npp], lead[:npp])
        if g:                        # another group's prefix is disjoint
            assert not np.intersect1d(used[b][:npp], used[0][:npp]).size
        others = np.concatenate([u for c, u in enumerate(used) if c != b])
        assert not np.intersect1d(used[b][npp:], others).size   # the suffix is private


@pytest.mark.parametrize("name", ["mla_b48", "mla_b48_ctl", "gqa_64k", "varlen_drafts"])
@pytest.mark.parametrize("batch", [1, 2, 4, 8, 16, 24, 48])
def test_bench_batch_scaling_fits_the_pool(name, batch):
    w = bench.batch_workload(name, batch)
    assert w.batch == batch and len(set(w.context_lens)) == 1
    assert w.context_lens[0] == CONFIGS[name].context_lens[0]
    assert w.pages_needed() <= w.pool_pages
    _tables(w)                       # raises if the pool were too small
