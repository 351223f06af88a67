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

Centroid variant (KVDrive, Fig 18 and Fig 19 vary the number of centroids,
2048 to 8192; the pages print no rule).  Reading used here, the plainest one
that produces exactly K entries:

  * the older positions of a head are partitioned into C clusters, each
    with a centroid key (the clustering itself happens before decode and is
    an input); members of a cluster are listed in ascending position order;
  * a cluster's score is the largest, over the head's query rows, of
    q_r . centroid, just as a position's score is for its key;
  * clusters are taken whole in descending score (ties to the lower cluster
    id) until K - window entries are covered; the cluster that crosses the
    count gives its lowest positions; members at or past L - window are
    ignored (they are in the window);
  * the window is kept and the list returned in ascending order.

Parity: pinned by tests/test_oracle_select.py (a pure-Python sort over brute
force scores on tiny inputs, exactly representable inputs with deliberate
ties, structural invariants; for the centroid variant a hand-worked
fixture, the reduction to the exact selection when every cluster is one
position whose centroid is its key, and structural invariants).
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


def centroid_scores(q, centroids, s: int, h: int, gqa: int):
    """fp64 scores of the C centroids of (s, h).  q: uint16 [B][Hq][D];
    centroids: uint16 bf16 bits [B][Hkv][C][D]."""
    C = bf16_to_f64(centroids[s, h])                   # [C][D]
    Q = bf16_to_f64(q[s, h * gqa:(h + 1) * gqa])       # [gqa][D]
    return (Q @ C.T).max(axis=0)                       # [C]


def select_clusters(cscore: np.ndarray, cl_start: np.ndarray, cl_pos: np.ndarray, L: int,
                    K: int, window: int) -> np.ndarray:
    """Indices (ascending, int32) chosen through the clusters of one head.

    cscore [C]; cluster c's members are cl_pos[cl_start[c]:cl_start[c+1]],
    ascending.  Requires the clusters to hold at least K - window positions
    below L - window."""
    assert 0 <= window <= K <= L
    n = L - window
    need = K - window
    C = len(cscore)
    order = np.lexsort((np.arange(C), -cscore))      # score desc, then cluster id asc
    chosen = []
    for c in order:
        if need == 0:
            break
        members = [int(t) for t in cl_pos[cl_start[c]:cl_start[c + 1]] if t < n]
        take = members[:need]
        chosen.extend(take)
        need -= len(take)
    assert need == 0, "the clusters do not cover K - window older positions"
    return np.concatenate([np.sort(np.array(chosen, dtype=np.int64)),
                           np.arange(n, L)]).astype(np.int32)
