"""Top-K selection of critical entries, stated plainly (test infrastructure).

KVDrive (Fig 1, Fig 7) attends, at each decode step, to a small set of
critical KV entries chosen by attention behaviour, together with a window of
recent entries (Fig 3: critical KV windows).  The pages do not print the
selection rule; the reading used here is the plainest exact one:

  * score of position t of KV head h = the largest, over the query rows r
    of h, of q_r . k_t (the softmax is monotone, so the scale does not
    matter; the largest row is the one that would give t the most weight);
  * the `window` most recent positions L-window .. L-1 are always kept;
  * the remaining K - window entries are the highest-scoring positions of
    0 .. L-window-1, ties going to the lower position;
  * the list is returned in ascending order.

Parity: pinned by tests/test_oracle_select.py (a pure-Python sort over brute
force scores on tiny inputs, exactly representable inputs with deliberate
ties, and structural invariants).
"""
from __future__ import annotations

import numpy as np

from . import pager as pg


def bf16_to_f64(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def scores(q, pool_k, spec: pg.PagerSpec, s: int, h: int):
    """fp64 scores of every retained position of (s, h).  q: uint16 [B][Hq][D]."""
    gqa = q.shape[1] // spec.hkv
    L = int(spec.lengths[s, h])
    D = pool_k.shape[-1]
    flat = pool_k.reshape(-1, D)
    rows = np.array([spec.physical_row(s, h, t) for t in range(L)], dtype=np.int64)
    K = bf16_to_f64(flat[rows])                       # [L][D]
    Q = bf16_to_f64(q[s, h * gqa:(h + 1) * gqa])      # [gqa][D]
    return (Q @ K.T).max(axis=0)                      # [L]


def select(score: np.ndarray, K: int, window: int) -> np.ndarray:
    """Indices (ascending, int32) chosen from the scores of one head."""
    L = len(score)
    assert 0 <= window <= K <= L
    n = L - window
    k = K - window
    cand = np.arange(n)
    # highest score first, then lower position first
    order = np.lexsort((cand, -score[:n]))
    chosen = np.sort(order[:k])
    return np.concatenate([chosen, np.arange(n, L)]).astype(np.int32)


def select_all(q, pool_k, spec: pg.PagerSpec, K: int, window: int):
    """[B][Hkv][K] index lists for the active sequences (inactive rows: -1),
    and the per-head scores used."""
    B, H = spec.bmax, spec.hkv
    out = np.full((B, H, K), -1, dtype=np.int32)
    sc = {}
    for s in range(B):
        if not spec.active[s]:
            continue
        for h in range(H):
            sc[(s, h)] = scores(q, pool_k, spec, s, h)
            out[s, h] = select(sc[(s, h)], K, window)
    return out, sc
