"""LDS bank behaviour of the stage-1 tile layouts, on the host (no GPU).

Bank model of gfx950: 64 banks of 4 bytes, bank = (byte address / 4) % 64
(rocm-libraries PR #10102, Motivation bank table), and 256 bytes served per
cycle, so a wave's read is served in phases that must each touch every bank
once (lanes reading the same address share the access).  Which lanes form a
phase was measured on MI355X with an LDS probe (per-lane address tables,
SQ_LDS_BANK_CONFLICT per pattern):

* 16-byte reads: four phases of 16 lanes; a phase is lane quads {0, 3} of a
  16-lane window w together with quads {1, 2} of window w ^ 1.  Every
  permutation inside one window was conflict-free; moving one lane onto
  another lane's bank conflicted exactly when the two were in one such phase.
* 8-byte reads: lanes 0-31 and lanes 32-63.

The calculator first reproduces the page's bank table and pad-choice figures
(whose counting is per whole wave or per first 16 lanes), then certifies the
access patterns the kernels use: the lane-to-address mapping is restated here
from the kernels' own layout rules (slot formulas, load orders) and checked
for full, disjoint coverage of the tile by the DMA and one touch per bank per
phase.
"""

import os

import numpy as np
import pytest

from tests.test_oracle import read_table


def phases(width):
    """Lane sets served together for reads of `width` bytes (measured)."""
    if width == 16:
        out = []
        for w in range(4):
            own = [16 * w + i for i in list(range(0, 4)) + list(range(12, 16))]
            partner = [16 * (w ^ 1) + i for i in range(4, 12)]
            out.append(own + partner)
        return out
    per = 256 // width
    return [list(range(p, p + per)) for p in range(0, 64, per)]


def test_phases_partition_the_wave():
    for width in (16, 8, 4):
        lanes = sorted(l for ph in phases(width) for l in ph)
        assert lanes == list(range(64)) and all(len(ph) == 256 // width for ph in phases(width))


def bank_histograms(byte_addrs, width):
    """Per phase, how many dword accesses each of the 64 banks takes (one
    access per distinct address: lanes reading the same address share it)."""
    out = []
    for ph in phases(width):
        h = np.zeros(64, dtype=int)
        for a in sorted({byte_addrs[l] for l in ph}):
            for d in range(width // 4):
                h[(a // 4 + d) % 64] += 1
        out.append(h)
    return out


def max_phase_depth(byte_addrs, width):
    return max(int(h.max()) for h in bank_histograms(byte_addrs, width))


# ---- the pages' figures ----

def qk_operand_addrs(D, rows_per_group, pitch):
    """Lane L reads 8 bf16 of key row L % 32 at column (L // 32) * 8; rows are
    packed rows_per_group to an LDS group of `pitch` elements."""
    out = []
    for L in range(64):
        row, col = L % 32, (L // 32) * 8
        elem = (row // rows_per_group) * pitch + (row % rows_per_group) * D + col
        out.append(elem * 2)
    return out


def test_reproduces_bank_table():
    txt = open(os.path.join(os.path.dirname(__file__), "golden", "rocmlib10102_lds_banks.txt")).read()
    rows = [ln.split() for ln in txt.splitlines() if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 5
    for name, D, rpg, pitch, banks, depth in rows:
        addrs = qk_operand_addrs(int(D), int(rpg), int(pitch))
        touched = set()
        for a in addrs:
            for d in range(4):
                touched.add((a // 4 + d) % 64)
        h = np.zeros(64, dtype=int)
        for a in addrs:
            for d in range(4):
                h[(a // 4 + d) % 64] += 1
        assert len(touched) == int(banks), name
        assert int(h.max()) == int(depth) and int(h[h > 0].min()) == int(depth), name


def test_reproduces_pad_choice():
    _, rows = read_table("rocmlib10102_phase_banks.txt")
    for r in rows:
        addrs = qk_operand_addrs(64, 2, 128 + r["pad"])[:16]
        starts = [(a // 4) % 64 for a in addrs]
        assert len(set(starts)) == r["distinct_start_banks"], r
        assert max(starts.count(s) for s in set(starts)) == r["repeats"], r


# ---- the MFMA stage-1 tile (32 keys, 16-byte slots) ----

def swz(k):
    return (-(k >> 2)) & 3


def swz_plain(k):
    return (k >> 2) & 3


def swz_bits_swapped(k):
    v = (k >> 2) & 3
    return ((v & 1) << 1) | (v >> 1)


def slot(k, c, s=swz):
    return (c >> 2) * 128 + 4 * k + ((c & 3) ^ s(k))


@pytest.mark.parametrize("dk", [64, 128, 256, 576])
def test_mfma_tile_dma_fills_every_slot_once(dk):
    kch = dk * 2 // 16
    seen = {}
    for i in range(kch // 2):
        for lane in range(64):
            key = (i & 1) * 16 + lane // 4
            chunk = (i >> 1) * 4 + ((lane & 3) ^ swz(key))
            assert slot(key, chunk) == i * 64 + lane
            seen[(key, chunk)] = seen.get((key, chunk), 0) + 1
    assert len(seen) == 32 * kch and set(seen.values()) == {1}


def qk_reads(kk, second_half, s=swz):
    out = []
    for lane in range(64):
        n, g = lane & 15, lane >> 4
        out.append(slot(16 * second_half + n, kk * 4 + g, s) * 16)
    return out


def pv_reads(dt, second_half, s=swz):
    out = []
    for lane in range(64):
        g, j, q4 = lane >> 4, (lane & 15) // 4, lane & 3
        rk = 16 * second_half + 4 * g + j
        out.append(slot(rk, 2 * dt + (q4 >> 1), s) * 16 + (q4 & 1) * 8)
    return out


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (256, 256), (576, 512)])
def test_mfma_tile_reads_conflict_free(dk, dv):
    for kk in range(dk // 32):
        for h in (0, 1):
            assert max_phase_depth(qk_reads(kk, h), 16) == 1, (kk, h)
    for dt in range(dv // 16):
        for h in (0, 1):
            assert max_phase_depth(pv_reads(dt, h), 8) == 1, (dt, h)


def test_other_swizzles_conflict():
    # planted: the plain (k/4)%4 swizzle doubles up both patterns; with its
    # two bits swapped the transpose reads are clean but Q.K is not (both
    # measured two-deep on MI355X, as predicted here)
    assert max_phase_depth(qk_reads(0, 0, swz_plain), 16) == 2
    assert max_phase_depth(pv_reads(0, 0, swz_plain), 8) == 2
    assert max_phase_depth(qk_reads(0, 0, swz_bits_swapped), 16) == 2
    assert max_phase_depth(pv_reads(0, 0, swz_bits_swapped), 8) == 1


def test_measured_probe_patterns():
    # the probe's findings, restated: contiguous and in-window permutations
    # are clean; lane b moved onto lane 0's bank conflicts for b in quads 1-2
    base = [(l // 16) * 4096 + (l % 16) * 16 for l in range(64)]
    assert max_phase_depth(base, 16) == 1
    for b, deep in ((1, 1), (2, 1), (4, 2), (8, 2), (12, 1), (17, 1), (20, 2), (24, 2), (28, 1),
                    (36, 2), (40, 2), (44, 1), (52, 2), (56, 2), (60, 1)):
        a = list(base)
        a[b] = (b // 16) * 4096
        assert max_phase_depth(a, 16) == deep, b


def test_pv_transpose_reads_cover_the_operand():
    # lane 16g + s addresses dims 4*(s%4).. of key 4g + s/4: over the two
    # reads and a 16-lane group's four 64-bit words, every (key, dim) pair of
    # the 32-key x 16-dim operand of one step appears exactly once
    for dt in (0, 1, 7, 31):
        cover = {}
        for h in (0, 1):
            for lane in range(64):
                g, j, q4 = lane >> 4, (lane & 15) // 4, lane & 3
                key = 16 * h + 4 * g + j
                c = 2 * dt + (q4 >> 1)
                assert slot(key, c) * 16 + (q4 & 1) * 8 == pv_reads(dt, h)[lane]
                for e in range(4):
                    dim = c * 8 + (q4 & 1) * 4 + e
                    cover[(key, dim)] = cover.get((key, dim), 0) + 1
        assert len(cover) == 32 * 16 and set(cover.values()) == {1}


# ---- the VALU stage-1 K tile (64 keys, groups of one load each) ----

GP = 64 * 16 + 16  # bytes per load group: 1 KB plus a 16-byte pad


@pytest.mark.parametrize("krb", [256])
def test_valu_k_tile_reads_conflict_free(krb):
    # four rows per load: load i holds keys i, 16+i, 32+i, 48+i; key t sits in
    # group t % 16 at row position t // 16
    kch = krb // 16
    for c in range(kch):
        addrs = [(t & 15) * GP + (t >> 4) * krb + c * 16 for t in range(64)]
        assert max_phase_depth(addrs, 16) == 1, c
