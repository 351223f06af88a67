"""Pins for the top-K selection oracle (CPU only)."""
import numpy as np
import pytest

from oracle import pager as pg
from oracle import select as sel
from workloads import f32_to_bf16_bits


def test_select_brute_force():
    rs = np.random.default_rng(0)
    for trial in range(200):
        L = int(rs.integers(1, 40))
        K = int(rs.integers(1, L + 1))
        window = int(rs.integers(0, K + 1))
        score = rs.integers(-3, 4, size=L).astype(np.float64)   # many ties
        got = sel.select(score, K, window).tolist()
        # brute force: rank candidates by (score desc, position asc) with a plain sort
        cands = sorted(range(L - window), key=lambda t: (-score[t], t))[:K - window]
        want = sorted(cands) + list(range(L - window, L))
        assert got == want


def test_select_structure():
    rs = np.random.default_rng(1)
    score = rs.standard_normal(1000)
    idx = sel.select(score, 100, 30)
    assert len(idx) == 100 and (np.diff(idx) > 0).all()
    assert idx[-30:].tolist() == list(range(970, 1000))
    chosen = idx[:70]
    rest = np.setdiff1d(np.arange(970), chosen)
    assert score[chosen].min() >= score[rest].max()


def _pager_with_keys(L, D=16, H=2, gqa=2):
    p = pg.PagerSpec(H, 1, 1, 64, 64, 16)
    assert p.alloc([0], np.array([[L] * H]), np.array([[L] * H])) == pg.OK
    return p


def test_scores_exact_on_representable_inputs():
    """q picks one dim with weight 1 (row 0) or 0.5 (row 1): every score is an
    exact bf16 value, so the fp64 oracle equals a hand computation."""
    H, gqa, D, L = 2, 2, 16, 50
    p = _pager_with_keys(L, D, H, gqa)
    pool = np.zeros((64, H, 16, D), np.float32)
    vals = np.arange(L, dtype=np.float32) % 7 - 3.0        # ties on purpose
    for t in range(L):
        page = p.page_table[0, 0, t // 16]
        pool[page, 0, t % 16, 3] = vals[t]
        pool[page, 1, t % 16, 5] = -vals[t]
    q = np.zeros((1, H * gqa, D), np.float32)
    q[0, 0, 3] = 1.0
    q[0, 1, 3] = 0.5
    q[0, 2, 5] = 0.25
    q[0, 3, 5] = 2.0
    qb, kb = f32_to_bf16_bits(q), f32_to_bf16_bits(pool)
    s0 = sel.scores(qb, kb, p, 0, 0)
    s1 = sel.scores(qb, kb, p, 0, 1)
    np.testing.assert_array_equal(s0, np.maximum(vals, 0.5 * vals))
    np.testing.assert_array_equal(s1, np.maximum(-0.25 * vals, -2.0 * vals))
    idx = sel.select(s0, 12, 4)
    assert idx.tolist()[-4:] == [46, 47, 48, 49]
    # value 3 occurs at t = 6, 13, 20, 27, 34, 41: the first 8 highest go to the
    # lowest positions (six 3s, then 2s at t = 5, 12)
    assert idx.tolist()[:8] == [5, 6, 12, 13, 20, 27, 34, 41]


# ---- centroid variant ------------------------------------------------------

import json  # noqa: E402
import os  # noqa: E402

CENT = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_centroids.json")))


def _csr(clusters):
    start = np.concatenate([[0], np.cumsum([len(c) for c in clusters])]).astype(np.int32)
    pos = np.concatenate([np.array(c, np.int32) for c in clusters]) if clusters else np.zeros(0, np.int32)
    return start, pos


def test_centroid_fixture():
    start, pos = _csr(CENT["clusters"])
    cs = np.array(CENT["cluster_scores"])
    for case in CENT["cases"]:
        got = sel.select_clusters(cs, start, pos, CENT["L"], case["K"], case["window"])
        assert got.tolist() == case["want"], case["note"]


def test_centroids_equal_exact_selection_for_singleton_clusters():
    """One position per cluster, centroid = that position's key: the cluster
    order is the position order by (score desc, position asc), so the result
    is the exact selection."""
    rs = np.random.default_rng(7)
    H, gqa, D = 2, 3, 16
    for trial in range(30):
        L = int(rs.integers(2, 60))
        p = pg.PagerSpec(H, 1, 1, 64, 64, 16)
        assert p.alloc([0], np.array([[L] * H]), np.array([[L] * H])) == pg.OK
        keys = rs.integers(-3, 4, size=(64, H, 16, D)).astype(np.float32)   # ties on purpose
        q = rs.integers(-2, 3, size=(1, H * gqa, D)).astype(np.float32)
        kb, qb = f32_to_bf16_bits(keys), f32_to_bf16_bits(q)
        for h in range(H):
            rows = [p.physical_row(0, h, t) for t in range(L)]
            cent = kb.reshape(-1, D)[rows][None, None].repeat(H, axis=1)   # [1][H][L][D]
            cs = sel.centroid_scores(qb, cent, 0, h, gqa)
            exact = sel.scores(qb, kb, p, 0, h)
            np.testing.assert_array_equal(cs, exact)
            K = int(rs.integers(1, L + 1))
            window = int(rs.integers(0, K + 1))
            start, pos = _csr([[t] for t in range(L)])
            assert sel.select_clusters(cs, start, pos, L, K, window).tolist() == \
                sel.select(exact, K, window).tolist()


def test_centroid_selection_structure():
    """Exactly K ascending entries with the window; the clusters fully taken
    score at least as high as every cluster left untouched."""
    rs = np.random.default_rng(8)
    for trial in range(100):
        L = int(rs.integers(5, 400))
        C = int(rs.integers(1, 40))
        assign = rs.integers(0, C, size=L)
        clusters = [sorted(np.nonzero(assign == c)[0].tolist()) for c in range(C)]
        start, pos = _csr(clusters)
        cs = rs.integers(-5, 6, size=C).astype(np.float64)
        K = int(rs.integers(1, L + 1))
        window = int(rs.integers(0, K + 1))
        got = sel.select_clusters(cs, start, pos, L, K, window)
        n = L - window
        assert len(got) == K and (np.diff(got) > 0).all()
        assert got[K - window:].tolist() == list(range(n, L))
        taken = set(got[:K - window].tolist())
        full = [c for c in range(C) if all(t in taken for t in clusters[c] if t < n)
                and any(t < n for t in clusters[c])]
        none = [c for c in range(C) if not any(t in taken for t in clusters[c] if t < n)
                and any(t < n for t in clusters[c])]
        if full and none:
            assert min(cs[full]) >= max(cs[none])
