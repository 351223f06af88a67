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
