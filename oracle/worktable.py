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
    so the slowest worker is within one page of the average;
  * tables in worker order (the share-aware plan, where a worker's first
    row may be another sequence's copy of a shared chunk): head_rows lists
    each head's rows, and the coverage checks apply to the table read
    through it; head_rows must be a permutation of the rows.  Shares there
    follow each worker's room after its first row, so the balance bound
    takes a slack of one page.  Workers whose first row runs in a launch of
    its own (skip[w] = 1: the share-aware plan's gang launch) are balanced
    without that row.

Parity: the checker is pinned by tests that feed it hand-made valid and
invalid tables (tests/test_oracle_worktable.py).
"""
from __future__ import annotations

import math

import numpy as np


def check(rows, worker_start, head_row_start, caps, active, page=16,
          balanced=True, head_rows=None, slack=0, skip=None):
    """rows: int [n][4] = (s*Hkv + h, t0, t1, _); worker_start: [W+1];
    head_row_start: [B*Hkv + 1]; head_rows: [n] row ids by head, or None
    when each head's rows are contiguous in the table.  Raises
    AssertionError on the first violated property; returns the per-worker
    page totals."""
    rows = np.asarray(rows).reshape(-1, 4)
    by_head = rows
    if head_rows is not None:
        head_rows = np.asarray(head_rows)
        assert len(head_rows) == len(rows)
        assert np.array_equal(np.sort(head_rows), np.arange(len(rows))), "head_rows is not a permutation"
        by_head = rows[head_rows]
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
            assert tuple(by_head[lo, :3]) == (sh, 0, 0), f"head {sh}: row {by_head[lo]}"
            continue
        t = 0
        for i in range(lo, hi):
            assert by_head[i, 0] == sh, f"row {i} belongs to {by_head[i, 0]} not {sh}"
            assert by_head[i, 1] == t, f"row {i} starts at {by_head[i, 1]}, expected {t}"
            assert by_head[i, 1] % page == 0
            assert by_head[i, 2] > by_head[i, 1]
            t = int(by_head[i, 2])
        assert t == cap, f"head {sh} covered to {t}, capacity {cap}"
    loads = []
    for w in range(len(worker_start) - 1):
        pages = 0
        first = int(worker_start[w])
        if skip is not None and skip[w]:
            assert first < int(worker_start[w + 1]), f"worker {w} skips a row it does not have"
            first += 1
        for i in range(first, int(worker_start[w + 1])):
            pages += math.ceil(rows[i, 2] / page) - rows[i, 1] // page
        loads.append(pages)
    if balanced and loads:
        total = sum(loads)
        bound = math.ceil(total / len(loads))
        for w, ld in enumerate(loads):
            assert ld <= bound + slack, f"worker {w}: {ld} pages > {bound} + {slack}"
    return loads
