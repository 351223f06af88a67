"""Pins for the integer parts of the oracle: grouping, pager, append,
coalescer and gather (CPU only)."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import pager as pg

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_pager.json")))


def _tiny(free_list_init=None):
    p = pg.PagerSpec(4, 2, 2, 64, 16, 16, free_list_init)
    caps = np.tile(np.array(GOLD["budgets"]), (2, 1))
    assert p.alloc([0, 1], caps, caps) == pg.OK
    return p


def test_tiny_identity_fixture():
    p = _tiny()
    g = GOLD["identity"]
    assert p.group_of_head.tolist() == GOLD["group_of_head"]
    assert p.slot_of_head.tolist() == GOLD["slot_of_head"]
    assert p.page_table.tolist() == g["page_table"]
    assert p.free_list().tolist() == g["free_list_after"]
    runs = pg.coalesce(p.page_table, p.n_pages, p.active)
    assert [list(r) for r in runs] == g["runs"]
    assert p.physical_row(1, 3, 37) == g["physical_row_s1_h3_t37"]
    assert p.free_seqs([0]) == pg.OK
    assert p.free_list().tolist() == g["after_free_seq0"]["free_list"]
    caps = np.array([g["realloc_seq0_budgets"]])
    assert p.alloc([0], caps) == pg.OK
    assert p.page_table[:, 0].tolist() == g["after_realloc_seq0"]["page_table_seq0"]
    runs = pg.coalesce(p.page_table, p.n_pages, p.active)
    assert [list(r) for r in runs] == g["after_realloc_seq0"]["runs"]


def test_tiny_scrambled_fixture():
    sc = GOLD["scrambled"]
    p = _tiny(np.array(sc["free_list_init"]))
    runs = pg.coalesce(p.page_table, p.n_pages, p.active)
    assert [list(r) for r in runs] == sc["runs"]


def test_physical_row_matches_layout_definition():
    """Row id = position of (page, slot, t % P) in [num_pages][G_h][P]."""
    p = _tiny(np.random.default_rng(0).permutation(64))
    for s in range(2):
        for h in range(4):
            for t in range(0, int(p.lengths[s, h]), 7):
                page = p.page_table[p.group_of_head[h], s, t // 16]
                want = np.ravel_multi_index((page, p.slot_of_head[h], t % 16), (64, 2, 16))
                assert p.physical_row(s, h, t) == want


def test_errors_are_all_or_nothing():
    p = pg.PagerSpec(4, 2, 4, 10, 8, 16)
    caps = np.array([[16, 16, 64, 64], [16, 16, 64, 64]])
    assert p.alloc([0, 1], caps) == pg.OK       # 2 * (1 + 4) = 10 pages
    snap = (p.page_table.copy(), p.free_list().copy(), p.active.copy())
    assert p.alloc([2], caps[:1]) == pg.E_NOPAGES
    assert p.alloc([0], caps[:1]) == pg.E_STATE
    assert p.alloc([1, 1], caps) == pg.E_ARG
    assert p.alloc([5], caps[:1]) == pg.E_ARG
    assert p.alloc([2], np.array([[16, 16, 64, 129]])) == pg.E_ARG   # > max_pages * P
    assert p.alloc([2], caps[:1], np.array([[17, 0, 0, 0]])) == pg.E_ARG
    assert p.free_seqs([3]) == pg.E_STATE
    assert p.free_seqs([0, 0]) == pg.E_ARG
    assert np.array_equal(snap[0], p.page_table) and np.array_equal(snap[1], p.free_list())
    assert np.array_equal(snap[2], p.active)


def test_append_capacity():
    p = pg.PagerSpec(2, 1, 2, 8, 4, 16)
    assert p.alloc([1], np.array([[17, 3]]), np.array([[15, 3]])) == pg.OK
    st_, pos = p.append_positions()
    assert st_ == pg.E_CAPACITY and pos is None        # head 1 is full
    assert p.lengths[1].tolist() == [15, 3]
    p2 = pg.PagerSpec(2, 1, 2, 8, 4, 16)
    assert p2.alloc([1], np.array([[17, 4]]), np.array([[15, 3]])) == pg.OK
    st_, pos = p2.append_positions()
    assert st_ == pg.OK and pos[1].tolist() == [15, 3] and p2.lengths[1].tolist() == [16, 4]


@settings(max_examples=60, deadline=None)
@given(st.data())
def test_pager_invariants(data):
    """Random Reserve/Trim sequences: pages are conserved, never shared, and
    trains rebuild every page table exactly and are maximal."""
    hkv, ng = 4, data.draw(st.sampled_from([1, 2, 4]))
    bmax, num_pages, max_pages = 6, 60, 8
    perm = data.draw(st.permutations(list(range(num_pages))))
    p = pg.PagerSpec(hkv, ng, bmax, num_pages, max_pages, 16, np.array(perm))
    for _ in range(data.draw(st.integers(1, 12))):
        if data.draw(st.booleans()):
            cands = [s for s in range(bmax) if not p.active[s]]
            if not cands:
                continue
            slots = data.draw(st.lists(st.sampled_from(cands), min_size=1, max_size=3, unique=True))
            caps = np.array([[data.draw(st.integers(0, max_pages * 16)) for _ in range(hkv)]
                             for _ in slots])
            before = (p.page_table.copy(), p.free_list().copy())
            rc = p.alloc(slots, caps)
            if rc != pg.OK:
                assert rc == pg.E_NOPAGES
                assert np.array_equal(before[0], p.page_table)
                assert np.array_equal(before[1], p.free_list())
        else:
            cands = [s for s in range(bmax) if p.active[s]]
            if not cands:
                continue
            slots = data.draw(st.lists(st.sampled_from(cands), min_size=1, max_size=3, unique=True))
            assert p.free_seqs(slots) == pg.OK
        used = p.page_table[p.page_table >= 0]
        assert len(set(used.tolist())) == len(used)
        assert sorted(used.tolist() + p.free_list().tolist()) == list(range(num_pages))
        for s in range(bmax):
            for g in range(ng):
                n = p.n_pages[g, s]
                assert (p.page_table[g, s, :n] >= 0).all() and (p.page_table[g, s, n:] == -1).all()
        runs = pg.coalesce(p.page_table, p.n_pages, p.active)
        rebuilt = np.full_like(p.page_table, -1)
        prev = None
        for (s, g, ph, n, lo) in runs:
            rebuilt[g, s, lo:lo + n] = np.arange(ph, ph + n)
            if prev is not None and prev[0] == s and prev[1] == g:
                assert prev[4] + prev[3] == lo
                assert prev[2] + prev[3] != ph, "adjacent trains could merge"
            prev = (s, g, ph, n, lo)
        assert np.array_equal(rebuilt, p.page_table)


def _coded_pool(p, D=8):
    """Pool whose row for logical (s, h, t) holds a code of (s, h, t), placed
    with numpy's multi-dimensional indexing."""
    pk = np.zeros((p.num_pages, p.g_h, p.P, D), np.uint16)
    pv = np.zeros_like(pk)
    for s in range(p.bmax):
        if not p.active[s]:
            continue
        for h in range(p.hkv):
            for t in range(int(p.lengths[s, h])):
                page = p.page_table[p.group_of_head[h], s, t // p.P]
                pk[page, p.slot_of_head[h], t % p.P, :3] = (s, h, t)
                pv[page, p.slot_of_head[h], t % p.P, :3] = (s + 100, h + 100, t + 100)
    return pk, pv


def test_gather_index_reads_requested_logical_rows():
    p = _tiny(np.random.default_rng(1).permutation(64))
    pk, pv = _coded_pool(p)
    rs = np.random.default_rng(2)
    idx = np.stack([np.stack([np.sort(rs.choice(int(p.lengths[s, h]), 8, replace=False))
                              for h in range(4)]) for s in range(2)]).astype(np.int32)
    sk, sv, phys = pg.gather_index(p, pk, pv, idx)
    for s in range(2):
        for h in range(4):
            for k in range(8):
                assert sk[s, h, k, :3].tolist() == [s, h, idx[s, h, k]]
                assert sv[s, h, k, :3].tolist() == [s + 100, h + 100, idx[s, h, k] + 100]


def test_gather_pages_reads_every_retained_row():
    p = _tiny(np.random.default_rng(3).permutation(64))
    pk, pv = _coded_pool(p)
    want = pg.gather_pages(p, pk, pv, None)
    for (s, h), (kr, vr, rows) in want.items():
        assert len(kr) == p.lengths[s, h]
        assert kr[:, :3].tolist() == [[s, h, t] for t in range(len(kr))]
