"""Pins for the work-table checker: it accepts hand-made valid tables and
rejects each kind of invalid one."""
import numpy as np
import pytest

from oracle import worktable as wt

CAPS = np.array([[64, 16], [0, 48]])
ACTIVE = np.array([True, True])


def _valid():
    # heads (0,0): 64 tokens, (0,1): 16, (1,0): 0 (one empty row), (1,1): 48;
    # two workers of 4 pages
    rows = [(0, 0, 32, 0), (0, 32, 64, 0), (1, 0, 16, 0), (2, 0, 0, 0), (3, 0, 16, 0), (3, 16, 48, 0)]
    # worker 0: rows 0,1 (4 pages); worker 1: rows 2..5 (1 + 0 + 1 + 2 pages)
    return np.array(rows), np.array([0, 2, 6]), np.array([0, 2, 3, 4, 6])


def test_accepts_valid():
    rows, ws, hrs = _valid()
    loads = wt.check(rows, ws, hrs, CAPS, ACTIVE)
    assert loads == [4, 4]


@pytest.mark.parametrize("mutate", ["gap", "overlap", "unaligned", "short", "foreign", "unbalanced",
                                    "empty_head_uncovered"])
def test_rejects_invalid(mutate):
    rows, ws, hrs = _valid()
    rows = rows.copy()
    if mutate == "gap":
        rows[1, 1] = 48
    elif mutate == "overlap":
        rows[1, 1] = 16
    elif mutate == "unaligned":
        rows[0, 2] = 33
        rows[1, 1] = 33
    elif mutate == "short":
        rows[5, 2] = 40
    elif mutate == "foreign":
        rows[2, 0] = 2
    elif mutate == "unbalanced":
        ws = np.array([0, 0, 6])
    elif mutate == "empty_head_uncovered":
        rows = np.delete(rows, 3, axis=0)
        ws = np.array([0, 2, 5])
        hrs = np.array([0, 2, 3, 3, 5])
    with pytest.raises(AssertionError):
        wt.check(rows, ws, hrs, CAPS, ACTIVE)


def _worker_ordered():
    # the valid table above, stored in worker order with the rows of head 3
    # split across the two workers: worker 0 runs (3, 16..48) first, then
    # head 0; worker 1 runs heads 1, 2 and (3, 0..16)
    rows = [(3, 16, 48, 0), (0, 0, 32, 0), (0, 32, 48, 0),
            (0, 48, 64, 0), (1, 0, 16, 0), (2, 0, 0, 0), (3, 0, 16, 0)]
    head_rows = [1, 2, 3, 4, 5, 6, 0]      # by head, in token order
    return np.array(rows), np.array([0, 3, 7]), np.array([0, 3, 4, 5, 7]), np.array(head_rows)


def test_accepts_worker_ordered_table_through_head_rows():
    rows, ws, hrs, hr = _worker_ordered()
    loads = wt.check(rows, ws, hrs, CAPS, ACTIVE, head_rows=hr, balanced=False)
    assert loads == [5, 3]
    # worker 0 holds one page above the ceiling of the mean (4): accepted
    # only with the slack
    with pytest.raises(AssertionError):
        wt.check(rows, ws, hrs, CAPS, ACTIVE, head_rows=hr, slack=0)
    wt.check(rows, ws, hrs, CAPS, ACTIVE, head_rows=hr, slack=1)


@pytest.mark.parametrize("mutate", ["no_index", "not_permutation", "token_order", "wrong_head"])
def test_rejects_bad_head_rows(mutate):
    rows, ws, hrs, hr = _worker_ordered()
    hr = hr.copy()
    if mutate == "no_index":
        hr = None                          # the table is not head-contiguous
    elif mutate == "not_permutation":
        hr[0] = 2
    elif mutate == "token_order":
        hr[5], hr[6] = hr[6], hr[5]        # head 3's rows out of token order
    elif mutate == "wrong_head":
        hr[3], hr[4] = hr[4], hr[3]        # a row of head 2 listed under head 1
    with pytest.raises(AssertionError):
        wt.check(rows, ws, hrs, CAPS, ACTIVE, head_rows=hr, slack=1)


def test_skip_balances_without_the_skipped_rows():
    # worker 0's first row (head 3, 16..48) runs in a launch of its own: the
    # remaining loads are 3 and 3, within the ceiling of their mean
    rows, ws, hrs, hr = _worker_ordered()
    loads = wt.check(rows, ws, hrs, CAPS, ACTIVE, head_rows=hr, skip=[1, 0])
    assert loads == [3, 3]
    with pytest.raises(AssertionError):            # a worker with no row cannot skip one
        wt.check(rows, np.array([0, 0, 7]), hrs, CAPS, ACTIVE, head_rows=hr, skip=[1, 0], balanced=False)
