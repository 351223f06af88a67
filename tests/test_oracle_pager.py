"""Pins for the integer parts of the oracle: grouping, pager, append,
coalescer and gather (CPU only)."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import pager as pg

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_pager.json")))
ALIAS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_alias.json")))
TIES = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_grouping_ties.json")))


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


def test_grouping_ties_fixture():
    """Tied budgets and capacities that differ between sequences: the
    grouping key (sum over the first Reserve) and its tie-break (lower head
    index) against hand-worked groups, pages, trains and rows."""
    T = TIES
    caps = np.array(T["caps"])
    assert caps.sum(axis=0).tolist() == T["budget_sum"]
    goh, soh, members = pg.group_heads(caps, T["num_groups"])
    assert goh.tolist() == T["group_of_head"]
    assert soh.tolist() == T["slot_of_head"]
    p = pg.PagerSpec(T["num_kv_heads"], T["num_groups"], 2, T["num_pages"], T["max_pages"], 16)
    assert p.alloc([0, 1], caps, caps) == pg.OK
    assert p.group_of_head.tolist() == T["group_of_head"]
    assert p.slot_of_head.tolist() == T["slot_of_head"]
    assert p.n_pages.T.tolist() == T["pages_per_seq_group"]
    assert p.page_table.tolist() == T["page_table"]
    fl = p.free_list().tolist()
    assert len(fl) == T["free_list_after_len"] and fl[:3] == T["free_list_after_front"]
    runs = pg.coalesce(p.page_table, p.n_pages, p.active)
    assert [list(r) for r in runs] == T["runs"]
    assert p.physical_row(0, 2, 37) == T["physical_row_s0_h2_t37"]
    assert p.physical_row(1, 3, 17) == T["physical_row_s1_h3_t17"]
    # the grouping stays fixed through a later Reserve
    R = T["after_free_seq0_realloc"]
    assert p.free_seqs([0]) == pg.OK
    assert p.free_list().tolist()[-len(R["free_list_after_free_tail"]):] == R["free_list_after_free_tail"]
    assert p.alloc([0], np.array([R["caps_seq0"]])) == pg.OK
    assert p.group_of_head.tolist() == R["group_of_head"]
    assert p.page_table[:, 0].tolist() == R["page_table_seq0"]


def _grouping_with(key_of, reverse_ties=False):
    """A deliberately wrong grouping rule (planted here, on the CPU) that
    differs from the oracle's only in its key or its tie-break."""
    def rule(caps, ng):
        caps = np.asarray(caps, dtype=np.int64)
        hkv = caps.shape[1]
        key = key_of(caps)
        tie = (lambda h: -h) if reverse_ties else (lambda h: h)
        order = sorted(range(hkv), key=lambda h: (int(key[h]), tie(h)))
        goh = np.zeros(hkv, dtype=np.int32)
        soh = np.zeros(hkv, dtype=np.int32)
        for rank, h in enumerate(order):
            goh[h], soh[h] = rank // (hkv // ng), rank % (hkv // ng)
        return goh, soh
    return rule


@pytest.mark.parametrize("name,rule", [
    ("reversed_tie_break", _grouping_with(lambda c: c.sum(axis=0), reverse_ties=True)),
    ("max_capacity_key", _grouping_with(lambda c: c.max(axis=0))),
    ("first_sequence_key", _grouping_with(lambda c: c[0])),
    ("last_sequence_key", _grouping_with(lambda c: c[-1])),
])
def test_grouping_fixture_rejects_wrong_rules(name, rule, monkeypatch):
    """Each plausible mistake in the grouping rule yields the groups the
    fixture works out for it, and so fails the fixture: planted into the
    oracle, it breaks test_grouping_ties_fixture."""
    T = TIES
    goh, soh = rule(np.array(T["caps"]), T["num_groups"])
    assert goh.tolist() == T["wrong_rules"][name]["group_of_head"]
    assert soh.tolist() == T["wrong_rules"][name]["slot_of_head"]
    assert (goh.tolist(), soh.tolist()) != (T["group_of_head"], T["slot_of_head"])
    planted = lambda caps, ng: (*rule(caps, ng), None)
    monkeypatch.setattr(pg, "group_heads", planted)
    with pytest.raises(AssertionError):
        test_grouping_ties_fixture()


def test_tiny_scrambled_fixture():
    sc = GOLD["scrambled"]
    p = _tiny(np.array(sc["free_list_init"]))
    runs = pg.coalesce(p.page_table, p.n_pages, p.active)
    assert [list(r) for r in runs] == sc["runs"]


def _alias_state():
    p = pg.PagerSpec(4, 2, 3, 64, 16, 16)
    b = np.array([ALIAS["slot0_budgets"]])
    assert p.alloc([0], b, b) == pg.OK
    return p


def _alias_call(p, a):
    return p.alias([a["slot"]], [a["src"]], np.array([a["share_pages"]]),
                   np.array([a["caps"]]), np.array([a["lens"]]))


def test_tiny_alias_fixture():
    p = _alias_state()
    assert _alias_call(p, ALIAS["alias"]) == pg.OK
    assert p.page_table[:, 2].tolist() == ALIAS["page_table_slot2"]
    assert p.free_list().tolist() == ALIAS["free_list_after_alias"]
    assert p.ref.tolist() == ALIAS["refcounts_after_alias"]
    runs = pg.coalesce(p.page_table, p.n_pages, p.active)
    assert [list(r) for r in runs] == ALIAS["runs_after_alias"]
    assert p.physical_row(2, 3, 37) == ALIAS["physical_row_s2_h3_t37"]
    assert p.physical_row(0, 3, 37) == ALIAS["physical_row_s0_h3_t37"]
    assert p.physical_row(2, 3, 85) == ALIAS["physical_row_s2_h3_t85"]
    assert p.lengths[2].tolist() == ALIAS["alias"]["lens"]
    assert p.free_seqs([0]) == pg.OK
    assert p.free_list().tolist() == ALIAS["free_list_after_trim_slot0"]
    assert p.free_seqs([2]) == pg.OK
    assert p.free_list().tolist() == ALIAS["free_list_after_trim_slot2"]
    assert (p.ref == 0).all()


def test_tiny_alias_errors_are_all_or_nothing():
    codes = {"E_ARG": pg.E_ARG, "E_STATE": pg.E_STATE, "E_NOPAGES": pg.E_NOPAGES}
    p = _alias_state()
    # the source must be live
    assert p.alias([2], [1], np.zeros((1, 2)), np.full((1, 4), 16), np.zeros((1, 4))) == pg.E_STATE
    assert _alias_call(p, ALIAS["alias"]) == pg.OK
    snap = (p.page_table.copy(), p.free_list().copy(), p.ref.copy(), p.lengths.copy(), p.active.copy())
    for name, case in ALIAS["errors_from_alias_state"].items():
        assert _alias_call(p, case) == codes[case["status"]], name
        assert np.array_equal(snap[0], p.page_table) and np.array_equal(snap[1], p.free_list())
        assert np.array_equal(snap[2], p.ref) and np.array_equal(snap[3], p.lengths)
        assert np.array_equal(snap[4], p.active)
    ok = ALIAS["shared_needs_25_of_31"]
    assert _alias_call(p, ok) == pg.OK
    assert len(p.free_list()) == ok["free_after"]


def test_alias_with_no_shared_pages_is_a_reserve():
    """share = 0 everywhere: the same page tables, lengths and free list as
    kv_alloc of the same capacities."""
    rng = np.random.default_rng(3)
    perm = rng.permutation(80)
    a = pg.PagerSpec(4, 2, 4, 80, 8, 16, perm)
    b = pg.PagerSpec(4, 2, 4, 80, 8, 16, perm)
    c0 = np.array([[16, 40, 100, 128]])
    assert a.alloc([0], c0, c0) == pg.OK and b.alloc([0], c0, c0) == pg.OK
    caps = np.array([[30, 7, 128, 90], [0, 0, 0, 16]])
    lens = np.array([[3, 7, 0, 90], [0, 0, 0, 1]])
    assert a.alias([3, 1], [0, 0], np.zeros((2, 2)), caps, lens) == pg.OK
    assert b.alloc([3, 1], caps, lens) == pg.OK
    assert np.array_equal(a.page_table, b.page_table)
    assert np.array_equal(a.free_list(), b.free_list())
    assert np.array_equal(a.lengths, b.lengths) and np.array_equal(a.ref, b.ref)


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


def _check_refcounts(p):
    """Counts equal the number of live entries mapping each page; pages in
    use and the free list partition the pool; the next append of every live
    head lands on a page that only it maps."""
    used = p.page_table[p.page_table >= 0]
    count = np.bincount(used, minlength=p.num_pages) if used.size else np.zeros(p.num_pages, int)
    assert np.array_equal(count, p.ref)
    free = p.free_list().tolist()
    assert len(set(free)) == len(free)
    assert sorted(set(used.tolist())) + [] == sorted(set(range(p.num_pages)) - set(free))
    for s in range(p.bmax):
        if not p.active[s]:
            continue
        for h in range(p.hkv):
            t = int(p.lengths[s, h])
            if t < p.caps[s, h]:
                page = p.page_table[p.group_of_head[h], s, t // p.P]
                assert p.ref[page] == 1, (s, h, t)


@settings(max_examples=100, deadline=None)
@given(st.data())
def test_pager_alias_invariants(data):
    """Random Reserve / Alias / Trim / append sequences keep the counts,
    the partition of the pool and the exclusivity of every page an append
    can write."""
    hkv, ng = 4, data.draw(st.sampled_from([1, 2, 4]))
    bmax, num_pages, max_pages = 6, 60, 8
    perm = data.draw(st.permutations(list(range(num_pages))))
    p = pg.PagerSpec(hkv, ng, bmax, num_pages, max_pages, 16, np.array(perm))
    for _ in range(data.draw(st.integers(1, 14))):
        op = data.draw(st.sampled_from(["alloc", "alias", "free", "append"]))
        idle = [s for s in range(bmax) if not p.active[s]]
        live = [s for s in range(bmax) if p.active[s]]
        if op == "alloc" and idle:
            s = data.draw(st.sampled_from(idle))
            caps = np.array([[data.draw(st.integers(0, max_pages * 16)) for _ in range(hkv)]])
            lens = np.array([[data.draw(st.just(int(c)) | st.integers(0, int(c))) for c in caps[0]]])
            rc = p.alloc([s], caps, lens)
            assert rc in (pg.OK, pg.E_NOPAGES)
        elif op == "alias" and idle and live:
            s = data.draw(st.sampled_from(idle))
            src = data.draw(st.sampled_from(live))
            share = np.zeros((1, ng), np.int64)
            caps = np.zeros((1, hkv), np.int64)
            lens = np.zeros((1, hkv), np.int64)
            for g in range(ng):
                members = [h for h in range(hkv) if p.group_of_head[h] == g]
                most = min(int(p.lengths[src, h]) for h in members) // 16
                share[0, g] = data.draw(st.integers(0, most + 1))   # one past the limit now and then
                for h in members:
                    caps[0, h] = data.draw(st.integers(min(16 * most, max_pages * 16), max_pages * 16))
                    lens[0, h] = data.draw(st.integers(min(16 * int(share[0, g]), int(caps[0, h])),
                                                       int(caps[0, h])))
            before = (p.page_table.copy(), p.free_list().copy(), p.ref.copy())
            rc = p.alias([s], [src], share, caps, lens)
            if rc == pg.OK:
                for g in range(ng):
                    k = int(share[0, g])
                    assert np.array_equal(p.page_table[g, s, :k], p.page_table[g, src, :k])
            else:
                assert rc in (pg.E_ARG, pg.E_NOPAGES)
                assert np.array_equal(before[0], p.page_table)
                assert np.array_equal(before[1], p.free_list())
                assert np.array_equal(before[2], p.ref)
        elif op == "free" and live:
            slots = data.draw(st.lists(st.sampled_from(live), min_size=1, max_size=3, unique=True))
            assert p.free_seqs(slots) == pg.OK
        elif op == "append" and live:
            if (p.lengths[p.active] < p.caps[p.active]).all():
                assert p.append_positions()[0] == pg.OK
        _check_refcounts(p)


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
