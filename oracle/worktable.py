"""What makes an ahead-of-time split-K work table valid (test infrastructure).

Tangram (Fig 4c, Fig 5, abstract) replaces uniform KV splits across thread
blocks, which leave stragglers when per-head lengths differ, with a balance
computed ahead of time from the static budgets.  Many tables are correct, so
the table is judged by properties rather than bit-exactly:

  * coverage: for every active (s, h), the rows of that head tile
    [0, cap[s][h]) exactly once, in order, and are contiguous in the table;
    a head with no capacity (inactive sequence, or a zero budget) is covered
    by exactly one empty row (t0 = t1 = 0), whose worker writes that head's
    zero output;
  * granularity: every row starts on a page boundary;
  * head index: head_row_start[s*Hkv + h] .. head_row_start[s*Hkv + h + 1]
    lists exactly that head's rows;
  * balance (balanced plans): no worker holds more pages than the ceiling
    of the mean over workers (a page counts once even if only partly used),
    so the slowest worker is within one page of the average.

Parity: the checker is pinned by tests that feed it hand-made valid and
invalid tables (tests/test_oracle_worktable.py).
"""
from __future__ import annotations

import math

import numpy as np


def check(rows, worker_start, head_row_start, caps, active, page=16,
          balanced=True):
    """rows: int [n][4] = (s*Hkv + h, t0, t1, _); worker_start: [W+1];
    head_row_start: [B*Hkv + 1].  Raises AssertionError on the first
    violated property; returns the per-worker page totals."""
    rows = np.asarray(rows).reshape(-1, 4)
    caps = np.asarray(caps)
    B, H = caps.shape
    n = int(worker_start[-1])
    assert worker_start[0] == 0 and n == len(rows)
    assert all(worker_start[i] <= worker_start[i + 1] for i in range(len(worker_start) - 1))
    assert len(head_row_start) == B * H + 1 and head_row_start[0] == 0
    assert int(head_row_start[-1]) == n
    for sh in range(B * H):
        s, h = divmod(sh, H)
        lo, hi = int(head_row_start[sh]), int(head_row_start[sh + 1])
        cap = int(caps[s, h]) if active[s] else 0
        if cap == 0:
            assert hi - lo == 1, f"head {sh} without capacity needs one empty row"
            assert tuple(rows[lo, :3]) == (sh, 0, 0), f"head {sh}: row {rows[lo]}"
            continue
        t = 0
        for i in range(lo, hi):
            assert rows[i, 0] == sh, f"row {i} belongs to {rows[i, 0]} not {sh}"
            assert rows[i, 1] == t, f"row {i} starts at {rows[i, 1]}, expected {t}"
            assert rows[i, 1] % page == 0
            assert rows[i, 2] > rows[i, 1]
            t = int(rows[i, 2])
        assert t == cap, f"head {sh} covered to {t}, capacity {cap}"
    loads = []
    for w in range(len(worker_start) - 1):
        pages = 0
        for i in range(int(worker_start[w]), int(worker_start[w + 1])):
            pages += math.ceil(rows[i, 2] / page) - rows[i, 1] // page
        loads.append(pages)
    if balanced and loads:
        total = sum(loads)
        bound = math.ceil(total / len(loads))
        for w, ld in enumerate(loads):
            assert ld <= bound, f"worker {w}: {ld} pages > {bound}"
    return loads
