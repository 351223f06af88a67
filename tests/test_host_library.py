"""Host side of libnupaged.so on the CPU: the library loads and exports the
header's symbols, and its pager, grouping, trains and split-K plan match the
oracle's statement bit-exactly (plans: by the work-table properties)."""
import json
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import non_uniform_paged_amd as nup
from oracle import pager as pg
from oracle import worktable as wt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "tiny_pager.json")))


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "nupaged.h")).read()
    declared = set(re.findall(r"^\s*(?:nup_status|void|const char \*)\s*\*?\s*(\w+)\s*\(", hdr, re.M))
    assert {"kv_alloc_groups", "kv_append", "kv_gather_compact", "attn_decode_nonuniform",
            "attn_decode_topk"} <= declared
    for name in declared:
        assert hasattr(nup._lib, name), name
    assert declared == set(nup.EXPORTED)


def _host_ctx(H=4, Hq=4, D=64, ng=2, B=2, num_pages=64, max_pages=16, fl=None, **kw):
    return nup.Context(num_kv_heads=H, num_q_heads=Hq, head_dim=D, num_groups=ng, max_batch=B,
                       num_pages=num_pages, max_pages=max_pages, free_list_init=fl, **kw)


def _state(ctx):
    return (nup.get_page_table(ctx), nup.get_free_list(ctx), nup.get_lengths(ctx),
            nup.get_groups(ctx), nup.get_runs(ctx))


def test_tiny_fixture_identity():
    ctx = _host_ctx()
    caps = np.tile(np.array(GOLD["budgets"]), (2, 1))
    goh = nup.kv_alloc_groups(ctx, [0, 1], caps, caps)
    g = GOLD["identity"]
    assert goh.tolist() == GOLD["group_of_head"]
    assert nup.get_groups(ctx)[1].tolist() == GOLD["slot_of_head"]
    assert nup.get_page_table(ctx).tolist() == g["page_table"]
    assert nup.get_free_list(ctx).tolist() == g["free_list_after"]
    assert nup.get_runs(ctx).tolist() == g["runs"]
    nup.kv_free_seqs(ctx, [0])
    assert nup.get_free_list(ctx).tolist() == g["after_free_seq0"]["free_list"]
    nup.kv_alloc_groups(ctx, [0], np.array([g["realloc_seq0_budgets"]]))
    assert nup.get_page_table(ctx)[:, 0].tolist() == g["after_realloc_seq0"]["page_table_seq0"]
    assert nup.get_runs(ctx).tolist() == g["after_realloc_seq0"]["runs"]


def test_grouping_ties_fixture_through_the_library():
    """The tied-budget grouping fixture through the C ABI: same groups, slots,
    page tables and trains, and the grouping stays fixed on a later Reserve."""
    T = json.load(open(os.path.join(ROOT, "tests", "golden", "tiny_grouping_ties.json")))
    ctx = _host_ctx(num_pages=T["num_pages"], max_pages=T["max_pages"])
    caps = np.array(T["caps"])
    goh = nup.kv_alloc_groups(ctx, [0, 1], caps, caps)
    assert goh.tolist() == T["group_of_head"]
    assert nup.get_groups(ctx)[1].tolist() == T["slot_of_head"]
    assert nup.get_page_table(ctx).tolist() == T["page_table"]
    assert nup.get_runs(ctx).tolist() == T["runs"]
    R = T["after_free_seq0_realloc"]
    nup.kv_free_seqs(ctx, [0])
    nup.kv_alloc_groups(ctx, [0], np.array([R["caps_seq0"]]))
    assert nup.get_groups(ctx)[0].tolist() == R["group_of_head"]
    assert nup.get_page_table(ctx)[:, 0].tolist() == R["page_table_seq0"]


def test_tiny_fixture_scrambled():
    sc = GOLD["scrambled"]
    ctx = _host_ctx(fl=sc["free_list_init"])
    caps = np.tile(np.array(GOLD["budgets"]), (2, 1))
    nup.kv_alloc_groups(ctx, [0, 1], caps, caps)
    assert nup.get_runs(ctx).tolist() == sc["runs"]


def test_tiny_alias_fixture_through_the_library():
    """The hand-worked Alias fixture, through the C ABI."""
    A = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_alias.json")))
    ctx = _host_ctx(B=3)
    b = np.array([A["slot0_budgets"]])
    nup.kv_alloc_groups(ctx, [0], b, b)
    a = A["alias"]
    assert nup.kv_alias(ctx, [2], [1], [[0, 0]], [[16] * 4], [[0] * 4],
                        raise_on_error=False) == nup.NUP_E_STATE
    nup.kv_alias(ctx, [a["slot"]], [a["src"]], [a["share_pages"]], [a["caps"]], [a["lens"]])
    assert nup.get_page_table(ctx)[:, 2].tolist() == A["page_table_slot2"]
    assert nup.get_free_list(ctx).tolist() == A["free_list_after_alias"]
    assert nup.get_refcounts(ctx).tolist() == A["refcounts_after_alias"]
    assert nup.get_runs(ctx).tolist() == A["runs_after_alias"]
    codes = {"E_ARG": nup.NUP_E_ARG, "E_STATE": nup.NUP_E_STATE, "E_NOPAGES": nup.NUP_E_NOPAGES}
    pt = nup.get_page_table(ctx)
    for name, e in A["errors_from_alias_state"].items():
        rc = nup.kv_alias(ctx, [e["slot"]], [e["src"]], [e["share_pages"]], [e["caps"]], [e["lens"]],
                          raise_on_error=False)
        assert rc == codes[e["status"]], name
        assert np.array_equal(nup.get_page_table(ctx), pt)
    nup.kv_free_seqs(ctx, [0])
    assert nup.get_free_list(ctx).tolist() == A["free_list_after_trim_slot0"]
    nup.kv_free_seqs(ctx, [2])
    assert nup.get_free_list(ctx).tolist() == A["free_list_after_trim_slot2"]
    assert not nup.get_refcounts(ctx).any()


def test_error_codes_and_atomicity():
    ctx = _host_ctx(H=4, ng=2, B=4, num_pages=10, max_pages=8)
    caps = np.array([[16, 16, 64, 64], [16, 16, 64, 64]])
    nup.kv_alloc_groups(ctx, [0, 1], caps)
    snap = _state(ctx)
    E = nup
    assert nup.kv_alloc_groups(ctx, [2], caps[:1], raise_on_error=False) == E.NUP_E_NOPAGES
    assert nup.kv_alloc_groups(ctx, [0], caps[:1], raise_on_error=False) == E.NUP_E_STATE
    assert nup.kv_alloc_groups(ctx, [1, 1], caps, raise_on_error=False) == E.NUP_E_ARG
    assert nup.kv_alloc_groups(ctx, [5], caps[:1], raise_on_error=False) == E.NUP_E_ARG
    assert nup.kv_alloc_groups(ctx, [2], np.array([[16, 16, 64, 129]]), raise_on_error=False) == E.NUP_E_ARG
    assert nup.kv_alloc_groups(ctx, [2], caps[:1], np.array([[17, 0, 0, 0]]),
                               raise_on_error=False) == E.NUP_E_ARG
    assert nup.kv_free_seqs(ctx, [3], raise_on_error=False) == E.NUP_E_STATE
    assert nup.kv_free_seqs(ctx, [0, 0], raise_on_error=False) == E.NUP_E_ARG
    after = _state(ctx)
    for a, b in zip(snap, after):
        if isinstance(a, tuple):
            for x, y in zip(a, b):
                assert np.array_equal(x, y)
        else:
            assert np.array_equal(a, b)
    # device calls on a host-only context are refused, not crashed
    assert nup.nup_commit(ctx, stream=0, raise_on_error=False) == E.NUP_E_STATE
    import torch
    assert nup.attn_decode_nonuniform_append(ctx, None, None, None, None, None, 1.0, torch.zeros(1, dtype=torch.uint8),
                                             stream=0, raise_on_error=False) == E.NUP_E_STATE
    # graph replays are reported only between commits: arguments first, then state
    st = nup._lib.nup_note_appends
    assert st(ctx.handle, 1, 1) == E.NUP_E_ARG          # one layer: -1 and 0 only
    assert st(ctx.handle, -2, 1) == E.NUP_E_ARG
    assert st(ctx.handle, 0, -1) == E.NUP_E_ARG
    assert st(ctx.handle, -1, 1) == E.NUP_E_STATE        # never committed
    assert np.array_equal(_state(ctx)[0], snap[0])


def test_bad_configs_rejected():
    with pytest.raises(nup.NupError):
        _host_ctx(H=4, Hq=12)          # GQA 3 unsupported
    with pytest.raises(nup.NupError):
        _host_ctx(H=4, ng=3)
    with pytest.raises(nup.NupError):
        _host_ctx(D=96)
    with pytest.raises(nup.NupError):
        _host_ctx(fl=[0] * 64)         # not a permutation


@settings(max_examples=80, deadline=None)
@given(st.data())
def test_pager_matches_oracle(data):
    """Random Reserve / Trim sequences give bit-identical pager state."""
    H = data.draw(st.sampled_from([2, 4, 8]))
    ng = data.draw(st.sampled_from([g for g in (1, 2, 4) if H % g == 0]))
    B, num_pages, max_pages = 6, 80, 8
    perm = np.array(data.draw(st.permutations(list(range(num_pages)))), np.int32)
    ctx = _host_ctx(H=H, Hq=H, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages, fl=perm,
                    num_workers=7)
    spec = pg.PagerSpec(H, ng, B, num_pages, max_pages, 16, perm)
    for step in range(data.draw(st.integers(1, 12))):
        op = "alloc" if step == 0 else data.draw(st.sampled_from(["alloc", "alias", "free"]))
        if op == "alloc":
            slots = data.draw(st.lists(st.integers(0, B - 1), min_size=1, max_size=3, unique=True))
            caps = np.array([[data.draw(st.integers(0, max_pages * 16)) for _ in range(H)] for _ in slots])
            lens = np.array([[data.draw(st.just(int(c)) | st.integers(0, int(c))) for c in row]
                             for row in caps])
            a = spec.alloc(slots, caps, lens)
            b = nup.kv_alloc_groups(ctx, slots, caps, lens, raise_on_error=False)
        elif op == "alias":
            # any slots and sources, shares up to one page past what the
            # lengths allow: the error paths are compared too
            idle = [x for x in range(B) if not spec.active[x]]
            pick = st.sampled_from(idle) if idle and data.draw(st.integers(0, 3)) else st.integers(0, B - 1)
            slots = data.draw(st.lists(pick, min_size=1, max_size=2, unique=True))
            live = [x for x in range(B) if spec.active[x] and x not in slots]
            srcs = [data.draw(st.sampled_from(live) if live else st.integers(0, B - 1)) for _ in slots]
            share = np.zeros((len(slots), ng), np.int64)
            caps = np.zeros((len(slots), H), np.int64)
            lens = np.zeros((len(slots), H), np.int64)
            for i, src in enumerate(srcs):
                for g in range(ng):
                    heads = [h for h in range(H) if spec.group_of_head is not None
                             and spec.group_of_head[h] == g]
                    most = min([int(spec.lengths[src, h]) // 16 for h in heads], default=0)
                    over = data.draw(st.integers(0, 3)) == 0          # now and then one page too many
                    share[i, g] = data.draw(st.integers(0, most + 1) if over else st.integers(0, most))
                    for h in heads or range(g * (H // ng), (g + 1) * (H // ng)):
                        caps[i, h] = data.draw(st.integers(min(16 * most, max_pages * 16), max_pages * 16))
                        lens[i, h] = data.draw(st.integers(min(16 * int(share[i, g]), int(caps[i, h])),
                                                           int(caps[i, h])))
            a = spec.alias(slots, srcs, share, caps, lens)
            b = nup.kv_alias(ctx, slots, srcs, share, caps, lens, raise_on_error=False)
        else:
            slots = data.draw(st.lists(st.integers(0, B - 1), min_size=1, max_size=3, unique=True))
            a = spec.free_seqs(slots)
            b = nup.kv_free_seqs(ctx, slots, raise_on_error=False)
        assert a == b
        assert np.array_equal(nup.get_page_table(ctx), spec.page_table)
        assert np.array_equal(nup.get_free_list(ctx), spec.free_list())
        assert np.array_equal(nup.get_refcounts(ctx), spec.ref)
        assert np.array_equal(nup.get_lengths(ctx), spec.lengths)
        runs = [tuple(r) for r in nup.get_runs(ctx).tolist()]
        assert runs == pg.coalesce(spec.page_table, spec.n_pages, spec.active)
        if spec.group_of_head is not None:
            g, s = nup.get_groups(ctx)
            assert np.array_equal(g, spec.group_of_head) and np.array_equal(s, spec.slot_of_head)
        rows, ws, hrs = nup.get_plan(ctx)
        wt.check(rows, ws, hrs, spec.caps, spec.active)


@settings(max_examples=25, deadline=None)
@given(st.data())
def test_layers_share_one_pager(data):
    """Several layers in one pager: grouping over (layer, head) pairs, page
    tables and lengths equal the oracle pager's over those pairs, and each
    layer's plan covers exactly that layer's heads."""
    NL = data.draw(st.sampled_from([2, 3, 4]))
    H = data.draw(st.sampled_from([2, 4]))
    V = NL * H
    ng = data.draw(st.sampled_from([g for g in (1, 2, 3, 4, 6, 8, 12) if V % g == 0]))
    B, num_pages, max_pages = 4, 200, 8
    perm = np.array(data.draw(st.permutations(list(range(num_pages)))), np.int32)
    ctx = _host_ctx(H=H, Hq=2 * H, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages, fl=perm,
                    num_workers=11, num_layers=NL)
    spec = pg.PagerSpec(V, ng, B, num_pages, max_pages, 16, perm)
    for step in range(data.draw(st.integers(1, 6))):
        if step == 0 or data.draw(st.booleans()):
            slots = data.draw(st.lists(st.integers(0, B - 1), min_size=1, max_size=2, unique=True))
            caps = np.array([[data.draw(st.integers(0, max_pages * 16)) for _ in range(V)] for _ in slots])
            lens = np.array([[data.draw(st.integers(0, int(c))) for c in row] for row in caps])
            assert spec.alloc(slots, caps, lens) == nup.kv_alloc_groups(ctx, slots, caps, lens,
                                                                       raise_on_error=False)
        else:
            slots = data.draw(st.lists(st.integers(0, B - 1), min_size=1, max_size=2, unique=True))
            assert spec.free_seqs(slots) == nup.kv_free_seqs(ctx, slots, raise_on_error=False)
        assert np.array_equal(nup.get_page_table(ctx), spec.page_table)
        assert np.array_equal(nup.get_lengths(ctx), spec.lengths)
        assert np.array_equal(nup.get_free_list(ctx), spec.free_list())
        if spec.group_of_head is not None:
            g, sl = nup.get_groups(ctx)
            assert np.array_equal(g, spec.group_of_head) and np.array_equal(sl, spec.slot_of_head)
        for layer in range(NL):
            nup.set_layer(ctx, layer)
            rows, ws, hrs = nup.get_plan(ctx)
            wt.check(rows, ws, hrs, spec.caps[:, layer * H:(layer + 1) * H], spec.active)
    with pytest.raises(nup.NupError):
        nup.set_layer(ctx, NL)


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen25_32b", "mixed_churn"])
def test_plan_on_config_shapes(name):
    import workloads as W
    w = W.CONFIGS[name]()
    ctx = _host_ctx(H=w.num_kv_heads, Hq=w.num_q_heads, D=w.head_dim, ng=w.num_groups,
                    B=w.batch, num_pages=w.num_pages, max_pages=int(w.caps.max() // 16 + 1),
                    num_workers=2048)
    nup.kv_alloc_groups(ctx, np.arange(w.batch), w.caps, w.lengths)
    rows, ws, hrs = nup.get_plan(ctx)
    loads = wt.check(rows, ws, hrs, w.caps, np.ones(w.batch, bool))
    assert max(loads) - min(loads) <= 1
    # the uniform split, for contrast, leaves stragglers on skewed budgets
    uctx = _host_ctx(H=w.num_kv_heads, Hq=w.num_q_heads, D=w.head_dim, ng=w.num_groups,
                     B=w.batch, num_pages=w.num_pages, max_pages=int(w.caps.max() // 16 + 1),
                     plan_mode=nup.PLAN_UNIFORM, uniform_splits=8)
    nup.kv_alloc_groups(uctx, np.arange(w.batch), w.caps, w.lengths)
    rows, ws, hrs = nup.get_plan(uctx)
    uloads = wt.check(rows, ws, hrs, w.caps, np.ones(w.batch, bool), balanced=False)
    assert max(uloads) >= max(loads)


def test_product_does_not_touch_the_oracle():
    pkg = os.path.dirname(nup.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                src = open(os.path.join(root, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "_liboracle" not in src, f


def _forked_ctx(w, plan_mode, num_workers=2048):
    """The forked-prefix batch on a host-only context: Reserve the sources,
    then Alias each fork onto the whole pages of its shared prefix."""
    ctx = _host_ctx(H=w.num_kv_heads, Hq=w.num_q_heads, D=w.head_dim, ng=w.num_groups,
                    B=w.batch, num_pages=w.num_pages, max_pages=int(w.caps.max() // 16 + 1),
                    num_workers=num_workers, plan_mode=plan_mode)
    src = w.extra["alias_src"]
    roots, forks = np.nonzero(src < 0)[0], np.nonzero(src >= 0)[0]
    goh = nup.kv_alloc_groups(ctx, roots, w.caps[roots], w.lengths[roots])
    share = np.zeros((len(forks), w.num_groups), np.int32)
    for g in range(w.num_groups):
        share[:, g] = w.extra["prefix_tokens"][forks][:, goh == g].min(axis=1) // 16
    nup.kv_alias(ctx, forks, src[forks], share, w.caps[forks], w.lengths[forks])
    return ctx, goh, forks, share


def test_shared_plan_equals_balanced_without_sharing():
    import workloads as W
    w = W.qwen25_32b()
    plans = []
    for mode in (nup.PLAN_BALANCED, nup.PLAN_SHARED):
        ctx = _host_ctx(H=w.num_kv_heads, Hq=w.num_q_heads, D=w.head_dim, ng=w.num_groups,
                        B=w.batch, num_pages=w.num_pages, max_pages=int(w.caps.max() // 16 + 1),
                        num_workers=2048, plan_mode=mode)
        nup.kv_alloc_groups(ctx, np.arange(w.batch), w.caps, w.lengths)
        plans.append(nup.get_plan(ctx) + (nup.get_plan_head_rows(ctx),))
    for a, b in zip(plans[0], plans[1]):
        assert np.array_equal(a, b)
    assert np.array_equal(plans[1][3], np.arange(len(plans[1][0])))


def test_shared_plan_on_forked_batch():
    """Every head's capacity is covered exactly once (read through
    head_rows), workers stay within one page of the balance bound, and each
    set of sharers reads its common prefix as gangs: the chunk is the first
    row of each sharer's worker, and a chunk's workers sit on one XCD
    (workgroups of 4 waves dealt to 8 XCDs in turn)."""
    import workloads as W
    w = W.qwen25_32b_prefix()
    ctx, goh, forks, share = _forked_ctx(w, nup.PLAN_SHARED)
    rows, ws, hrs = nup.get_plan(ctx)
    hr = nup.get_plan_head_rows(ctx)
    gangs, skip = nup.get_plan_gangs(ctx)
    B, H = w.batch, w.num_kv_heads
    # the main launch, without the rows the gang launch runs, is balanced
    loads = wt.check(rows, ws, hrs, w.caps, np.ones(B, bool), head_rows=hr, slack=1, skip=skip)
    bctx, *_ = _forked_ctx(w, nup.PLAN_BALANCED)
    brows, bws, bhrs = nup.get_plan(bctx)
    bloads = wt.check(brows, bws, bhrs, w.caps, np.ones(B, bool))
    gang_pages = sum(int(rows[r, 2] - rows[r, 1]) // 16 for r in gangs.reshape(-1))
    assert sum(loads) + gang_pages == sum(bloads)
    # gang workgroups: four consecutive workers (one workgroup), each running
    # its first row there, all four rows one chunk of one head's shared pages
    assert len(gangs) > 0 and int(skip.sum()) == 4 * len(gangs)
    for blk in gangs:
        wk = [int(np.searchsorted(ws, r, side="right") - 1) for r in blk]
        assert wk[0] % 4 == 0 and wk == list(range(wk[0], wk[0] + 4))
        assert all(ws[x] == r and skip[x] == 1 for x, r in zip(wk, blk))
        assert len({tuple(rows[r, 1:3]) for r in blk}) == 1
        assert len({int(rows[r, 0]) % H for r in blk}) == 1
        assert len({int(rows[r, 0]) // H for r in blk}) == 4
    first = np.zeros(len(rows), bool)
    first[ws[:-1][ws[:-1] < ws[1:]]] = True
    worker_of = np.repeat(np.arange(len(ws) - 1), np.diff(ws))
    xcd = (worker_of // 4) % 8
    src = w.extra["alias_src"]
    n_gang_rows = 0
    for s0 in np.nonzero(src < 0)[0]:
        for h in range(H):
            g = goh[h]
            members = [s0] + [f for i, f in enumerate(forks) if src[f] == s0 and share[i, g] > 0]
            if len(members) < 2:
                continue
            common = min(int(share[i, g]) for i, f in enumerate(forks) if src[f] == s0 and share[i, g] > 0)
            common = min(common, min(int(w.caps[m, hh]) // 16 for m in members
                                     for hh in range(H) if goh[hh] == g))
            chunks = None
            for m in members:
                sh = m * H + h
                mine = [int(r) for r in hr[hrs[sh]:hrs[sh + 1]] if rows[r, 2] <= common * 16]
                assert sum(rows[r, 2] - rows[r, 1] for r in mine) == common * 16
                assert all(first[r] for r in mine)
                spans = [(int(rows[r, 1]), int(rows[r, 2])) for r in mine]
                if chunks is None:
                    chunks = {sp: [] for sp in spans}
                assert set(spans) == set(chunks)
                for r in mine:
                    chunks[(int(rows[r, 1]), int(rows[r, 2]))].append(xcd[r])
                n_gang_rows += len(mine)
            for span, xs in chunks.items():
                assert len(set(xs)) == 1, (s0, h, span, xs)
    assert n_gang_rows > len(forks)


@settings(max_examples=30, deadline=None)
@given(st.data())
def test_shared_plan_random_forks(data):
    """Random forks (some of forks), layers, groups (spanning layers) and
    worker counts: every layer's shared plan covers each of its heads exactly
    once, within one page of balance."""
    H = 4
    NL = data.draw(st.sampled_from([1, 2, 3]))
    V = NL * H
    ng = data.draw(st.sampled_from([g for g in (1, 2, 3, 4, 6, 8, 12) if V % g == 0]))
    B, num_pages, max_pages = 8, 400 * NL, 12
    W_ = data.draw(st.sampled_from([3, 7, 16, 37, 64]))
    D = data.draw(st.sampled_from([64, 128]))       # head_dim 128 may add gang workgroups
    ctx = _host_ctx(H=H, Hq=2 * H, D=D, ng=ng, B=B, num_pages=num_pages, max_pages=max_pages,
                    num_workers=W_, plan_mode=nup.PLAN_SHARED, num_layers=NL)
    spec = pg.PagerSpec(V, ng, B, num_pages, max_pages, 16, None)
    n_src = data.draw(st.integers(1, 3))
    lens = np.array([[data.draw(st.integers(16, 150)) for _ in range(V)] for _ in range(n_src)])
    caps = lens + 16
    assert spec.alloc(list(range(n_src)), caps, lens) == nup.kv_alloc_groups(ctx, list(range(n_src)), caps, lens,
                                                                              raise_on_error=False)
    slot = n_src
    for _ in range(data.draw(st.integers(0, B - n_src))):
        s0 = data.draw(st.integers(0, slot - 1))
        if not spec.active[s0]:
            continue
        goh = spec.group_of_head
        most = [min(int(spec.lengths[s0, h]) for h in range(V) if goh[h] == g) // 16 for g in range(ng)]
        sh = [data.draw(st.integers(0, m)) for m in most]
        fl = np.array([[sh[goh[h]] * 16 + data.draw(st.integers(0, 40)) for h in range(V)]])
        fc = fl + data.draw(st.integers(0, 20))
        a = spec.alias([slot], [s0], [sh], fc, fl)
        b = nup.kv_alias(ctx, [slot], [s0], [sh], fc, fl, raise_on_error=False)
        assert a == b
        slot += 1
    if data.draw(st.booleans()):
        victim = data.draw(st.integers(0, slot - 1))
        if spec.active[victim]:
            assert spec.free_seqs([victim]) == nup.kv_free_seqs(ctx, [victim], raise_on_error=False)
    for layer in range(NL):
        nup.set_layer(ctx, layer)
        rows, ws, hrs = nup.get_plan(ctx)
        hr = nup.get_plan_head_rows(ctx)
        gangs, skip = nup.get_plan_gangs(ctx)
        wt.check(rows, ws, hrs, spec.caps[:, layer * H:(layer + 1) * H], spec.active, head_rows=hr, slack=1,
                 skip=skip)


def test_plan_gangs_only_for_shared_plan_at_head_dim_128():
    """The gang launch exists only under the share-aware plan with head_dim
    128 and whole workgroups of workers; otherwise no workgroup is listed and
    no worker skips a row (the forked batch at 2048 workers has both)."""
    import workloads as W
    w = W.qwen25_32b_prefix()
    for mode, expect in ((nup.PLAN_BALANCED, False), (nup.PLAN_SHARED, True)):
        ctx, *_ = _forked_ctx(w, mode)
        gangs, skip = nup.get_plan_gangs(ctx)
        assert (len(gangs) > 0) == expect and (int(skip.sum()) > 0) == expect
    for D, workers in ((64, 2048), (128, 2044)):
        ctx = _host_ctx(H=w.num_kv_heads, Hq=w.num_q_heads, D=D, ng=w.num_groups, B=w.batch,
                        num_pages=w.num_pages, max_pages=int(w.caps.max() // 16 + 1),
                        num_workers=workers, plan_mode=nup.PLAN_SHARED)
        src = w.extra["alias_src"]
        roots, forks = np.nonzero(src < 0)[0], np.nonzero(src >= 0)[0]
        goh = nup.kv_alloc_groups(ctx, roots, w.caps[roots], w.lengths[roots])
        share = np.zeros((len(forks), w.num_groups), np.int32)
        for g in range(w.num_groups):
            share[:, g] = w.extra["prefix_tokens"][forks][:, goh == g].min(axis=1) // 16
        nup.kv_alias(ctx, forks, src[forks], share, w.caps[forks], w.lengths[forks])
        gangs, skip = nup.get_plan_gangs(ctx)
        assert len(gangs) == 0 and not skip.any(), (D, workers)
        rows, ws, hrs = nup.get_plan(ctx)
        wt.check(rows, ws, hrs, w.caps, np.ones(w.batch, bool), head_rows=nup.get_plan_head_rows(ctx), slack=1)
