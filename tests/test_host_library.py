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


def test_tiny_fixture_scrambled():
    sc = GOLD["scrambled"]
    ctx = _host_ctx(fl=sc["free_list_init"])
    caps = np.tile(np.array(GOLD["budgets"]), (2, 1))
    nup.kv_alloc_groups(ctx, [0, 1], caps, caps)
    assert nup.get_runs(ctx).tolist() == sc["runs"]


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


def test_bad_configs_rejected():
    with pytest.raises(nup.NupError):
        _host_ctx(H=4, Hq=12)          # GQA 3 unsupported
    with pytest.raises(nup.NupError):
        _host_ctx(H=4, ng=3)
    with pytest.raises(nup.NupError):
        _host_ctx(D=96)
    with pytest.raises(nup.NupError):
        _host_ctx(fl=[0] * 64)         # not a permutation


@settings(max_examples=40, deadline=None)
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
    for _ in range(data.draw(st.integers(1, 10))):
        if data.draw(st.booleans()):
            slots = data.draw(st.lists(st.integers(0, B - 1), min_size=1, max_size=3, unique=True))
            caps = np.array([[data.draw(st.integers(0, max_pages * 16)) for _ in range(H)] for _ in slots])
            lens = np.array([[data.draw(st.integers(0, int(c))) for c in row] for row in caps])
            a = spec.alloc(slots, caps, lens)
            b = nup.kv_alloc_groups(ctx, slots, caps, lens, raise_on_error=False)
        else:
            slots = data.draw(st.lists(st.integers(0, B - 1), min_size=1, max_size=3, unique=True))
            a = spec.free_seqs(slots)
            b = nup.kv_free_seqs(ctx, slots, raise_on_error=False)
        assert a == b
        assert np.array_equal(nup.get_page_table(ctx), spec.page_table)
        assert np.array_equal(nup.get_free_list(ctx), spec.free_list())
        assert np.array_equal(nup.get_lengths(ctx), spec.lengths)
        runs = [tuple(r) for r in nup.get_runs(ctx).tolist()]
        assert runs == pg.coalesce(spec.page_table, spec.n_pages, spec.active)
        if spec.group_of_head is not None:
            g, s = nup.get_groups(ctx)
            assert np.array_equal(g, spec.group_of_head) and np.array_equal(s, spec.slot_of_head)
        rows, ws, hrs = nup.get_plan(ctx)
        wt.check(rows, ws, hrs, spec.caps, spec.active)


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
