"""Integer and data-movement parts of the path, stated plainly (test infrastructure).

Parity: bit-exact.  Every function here is pinned by tests/test_oracle_pager.py
(a hand-worked fixture for the Tiny configuration, conservation and
exclusivity invariants, all-or-nothing failure, and round trips that rebuild
the page table from the runs).

Policy (the pages fix the mechanisms, not their tie-breaks; these readings
are the plainest ones and are listed with the others in the design notes):
  * Head grouping -- Tangram, Fig 8 / abstract (heads with similar retention
    share an independent page table).  Heads are ordered by their budget,
    the sum over the first allocation's sequences of their capacities, ties
    by head index, and cut into equal groups in that order; a head's slot in
    its page is its position inside its group.
  * Pages per (sequence, group): the group's largest capacity, in pages
    (one page table per group, sized to the group's most demanding head).
  * Block pager -- KV-RM, Fig 3 (Reserve / Trim / Alias edits).  A FIFO
    free list, initialised to a given permutation (or 0..N-1).  Reserve pops
    from the front for the sequences in call order, groups in order, logical
    pages in order; it is all-or-nothing.  Every physical page carries a
    count of the page-table entries that map it.  Alias is a Reserve whose
    first share[g] logical pages of group g map the pages a live source
    sequence holds there (their counts grow by one) instead of popping new
    ones; shared pages must be full in both sequences, so no append ever
    writes to them.  Trim drops a sequence's references in (group, logical
    page) order and pushes a page to the back when its count reaches zero.
  * Append -- the decode step writes the new token at logical slot L and
    then L grows by one; a fixed budget means L == capacity is an error.
  * Trains -- KV-RM, Fig 3 (descriptor merging into few large transfers):
    maximal runs of logical pages whose physical pages are consecutive,
    per (sequence, group), in (sequence, group, logical page) order.
"""
from __future__ import annotations

import collections
import math
from typing import Optional

import numpy as np

OK, E_ARG, E_NOPAGES, E_CAPACITY, E_STATE, E_HIP, E_INDEX = range(7)


def group_heads(caps: np.ndarray, num_groups: int):
    """caps: int [n][Hkv] capacities of the first allocation.

    Returns (group_of_head[Hkv], slot_of_head[Hkv], members[n_g][G_h])."""
    caps = np.asarray(caps, dtype=np.int64)
    hkv = caps.shape[1]
    g_h = hkv // num_groups
    key = caps.sum(axis=0)
    order = sorted(range(hkv), key=lambda h: (int(key[h]), h))
    group_of_head = np.zeros(hkv, dtype=np.int32)
    slot_of_head = np.zeros(hkv, dtype=np.int32)
    members = [[0] * g_h for _ in range(num_groups)]
    for rank, h in enumerate(order):
        group_of_head[h] = rank // g_h
        slot_of_head[h] = rank % g_h
        members[rank // g_h][rank % g_h] = h
    return group_of_head, slot_of_head, members


class PagerSpec:
    """The block pager with head-group page tables."""

    def __init__(self, num_kv_heads: int, num_groups: int, max_batch: int,
                 num_pages: int, max_pages: int, page_size: int = 16,
                 free_list_init: Optional[np.ndarray] = None):
        self.hkv, self.ng, self.bmax = num_kv_heads, num_groups, max_batch
        self.num_pages, self.max_pages, self.P = num_pages, max_pages, page_size
        self.g_h = num_kv_heads // num_groups
        init = range(num_pages) if free_list_init is None else [int(x) for x in free_list_init]
        self.free = collections.deque(init)
        self.page_table = np.full((num_groups, max_batch, max_pages), -1, dtype=np.int32)
        self.n_pages = np.zeros((num_groups, max_batch), dtype=np.int32)
        self.lengths = np.zeros((max_batch, num_kv_heads), dtype=np.int32)
        self.caps = np.zeros((max_batch, num_kv_heads), dtype=np.int32)
        self.active = np.zeros(max_batch, dtype=bool)
        self.ref = np.zeros(num_pages, dtype=np.int32)
        self.group_of_head = None
        self.slot_of_head = None

    # ---- Reserve ----------------------------------------------------------
    def alloc(self, slots, caps, lengths=None) -> int:
        slots = [int(s) for s in slots]
        caps = np.asarray(caps, dtype=np.int64).reshape(len(slots), self.hkv)
        lengths = (np.zeros_like(caps) if lengths is None else
                   np.asarray(lengths, dtype=np.int64).reshape(len(slots), self.hkv))
        if len(slots) == 0:
            return OK
        if len(set(slots)) != len(slots) or any(s < 0 or s >= self.bmax for s in slots):
            return E_ARG
        if (caps < 0).any() or (caps > self.max_pages * self.P).any():
            return E_ARG
        if (lengths < 0).any() or (lengths > caps).any():
            return E_ARG
        if any(self.active[s] for s in slots):
            return E_STATE
        if self.group_of_head is None:
            goh, soh, _ = group_heads(caps, self.ng)
        else:
            goh, soh = self.group_of_head, self.slot_of_head
        need = np.zeros((len(slots), self.ng), dtype=np.int64)
        for i in range(len(slots)):
            for g in range(self.ng):
                members = [h for h in range(self.hkv) if goh[h] == g]
                need[i, g] = math.ceil(max(int(caps[i, h]) for h in members) / self.P)
        if need.sum() > len(self.free):
            return E_NOPAGES
        self.group_of_head, self.slot_of_head = goh, soh
        for i, s in enumerate(slots):
            for g in range(self.ng):
                for j in range(int(need[i, g])):
                    self.page_table[g, s, j] = self.free.popleft()
                    self.ref[self.page_table[g, s, j]] = 1
                self.n_pages[g, s] = need[i, g]
            self.caps[s] = caps[i]
            self.lengths[s] = lengths[i]
            self.active[s] = True
        return OK

    # ---- Alias --------------------------------------------------------------
    def alias(self, slots, src_slots, share, caps, lengths) -> int:
        """Reserve slots[i] with its first share[i][g] logical pages of every
        group g mapped to the pages src_slots[i] holds there.

        Checks, in order: argument ranges (E_ARG); slots inactive and sources
        active (E_STATE); for every head h of group g, share*P within both the
        new length and the source's current length (E_ARG); enough free pages
        for the unshared rest (E_NOPAGES)."""
        slots = [int(s) for s in slots]
        src_slots = [int(s) for s in src_slots]
        n = len(slots)
        caps = np.asarray(caps, dtype=np.int64).reshape(n, self.hkv)
        lengths = np.asarray(lengths, dtype=np.int64).reshape(n, self.hkv)
        share = np.asarray(share, dtype=np.int64).reshape(n, self.ng)
        if n == 0:
            return OK
        if len(src_slots) != n or len(set(slots)) != n:
            return E_ARG
        if any(s < 0 or s >= self.bmax for s in slots + src_slots):
            return E_ARG
        if set(slots) & set(src_slots):
            return E_ARG
        if (caps < 0).any() or (caps > self.max_pages * self.P).any():
            return E_ARG
        if (lengths < 0).any() or (lengths > caps).any() or (share < 0).any():
            return E_ARG
        if any(self.active[s] for s in slots) or not all(self.active[s] for s in src_slots):
            return E_STATE
        goh = self.group_of_head
        for i in range(n):
            for h in range(self.hkv):
                tokens = int(share[i, goh[h]]) * self.P
                if tokens > lengths[i, h] or tokens > self.lengths[src_slots[i], h]:
                    return E_ARG
        need = np.zeros((n, self.ng), dtype=np.int64)
        for i in range(n):
            for g in range(self.ng):
                members = [h for h in range(self.hkv) if goh[h] == g]
                need[i, g] = math.ceil(max(int(caps[i, h]) for h in members) / self.P)
        if (need - share).sum() > len(self.free):
            return E_NOPAGES
        for i, s in enumerate(slots):
            src = src_slots[i]
            for g in range(self.ng):
                for j in range(int(need[i, g])):
                    if j < share[i, g]:
                        page = int(self.page_table[g, src, j])
                        self.ref[page] += 1
                    else:
                        page = self.free.popleft()
                        self.ref[page] = 1
                    self.page_table[g, s, j] = page
                self.n_pages[g, s] = need[i, g]
            self.caps[s] = caps[i]
            self.lengths[s] = lengths[i]
            self.active[s] = True
        return OK

    # ---- Trim -------------------------------------------------------------
    def free_seqs(self, slots) -> int:
        slots = [int(s) for s in slots]
        if len(set(slots)) != len(slots) or any(s < 0 or s >= self.bmax for s in slots):
            return E_ARG
        if any(not self.active[s] for s in slots):
            return E_STATE
        for s in slots:
            for g in range(self.ng):
                for j in range(int(self.n_pages[g, s])):
                    page = int(self.page_table[g, s, j])
                    self.ref[page] -= 1
                    if self.ref[page] == 0:
                        self.free.append(page)
                    self.page_table[g, s, j] = -1
                self.n_pages[g, s] = 0
            self.caps[s] = 0
            self.lengths[s] = 0
            self.active[s] = False
        return OK

    # ---- the decode step's write -------------------------------------------
    def append_positions(self):
        """(status, positions[B][Hkv]) for one appended token per active head."""
        pos = self.lengths.copy()
        act = self.active
        if (self.lengths[act] >= self.caps[act]).any():
            return E_CAPACITY, None
        self.lengths[act] += 1
        return OK, pos

    def physical_row(self, s: int, h: int, t: int) -> int:
        """Row id in the pool viewed as [num_pages * G_h * P] rows of D."""
        g = int(self.group_of_head[h])
        page = int(self.page_table[g, s, t // self.P])
        return (page * self.g_h + int(self.slot_of_head[h])) * self.P + t % self.P

    def free_list(self) -> np.ndarray:
        return np.array(self.free, dtype=np.int32)


def coalesce(page_table: np.ndarray, n_pages: np.ndarray, active: np.ndarray):
    """Trains: list of (s, g, phys_start, n_pages, logical_start)."""
    runs = []
    ng, bmax, _ = page_table.shape
    for s in range(bmax):
        if not active[s]:
            continue
        for g in range(ng):
            n = int(n_pages[g, s])
            i = 0
            while i < n:
                start = i
                while i + 1 < n and page_table[g, s, i + 1] == page_table[g, s, i] + 1:
                    i += 1
                runs.append((s, g, int(page_table[g, s, start]), i - start + 1, start))
                i += 1
    return runs


def gather_index(pager: PagerSpec, pool_k, pool_v, idx):
    """Index mode: stage[s][h][k] = row of logical position idx[s][h][k].

    pool_*: uint16 [num_pages][G_h][P][D]; idx: int32 [B][Hkv][K].
    Returns (stage_k, stage_v, phys) for active sequences (inactive rows 0,
    phys -1)."""
    B, H, K = idx.shape
    D = pool_k.shape[-1]
    flat_k = pool_k.reshape(-1, D)
    flat_v = pool_v.reshape(-1, D)
    sk = np.zeros((B, H, K, D), dtype=np.uint16)
    sv = np.zeros((B, H, K, D), dtype=np.uint16)
    phys = np.full((B, H, K), -1, dtype=np.int64)
    for s in range(B):
        if not pager.active[s]:
            continue
        for h in range(H):
            for k in range(K):
                row = pager.physical_row(s, h, int(idx[s, h, k]))
                phys[s, h, k] = row
                sk[s, h, k] = flat_k[row]
                sv[s, h, k] = flat_v[row]
    return sk, sv, phys


def gather_pages(pager: PagerSpec, pool_k, pool_v, row_off):
    """Page mode: stage[row_off[s][h] + t] = row (s, h, t) for t < L[s][h].

    Returns a dict {(s, h): (k_rows, v_rows, phys_rows)} of what must land at
    each (s, h)'s offset; padding between heads is unspecified."""
    D = pool_k.shape[-1]
    flat_k = pool_k.reshape(-1, D)
    flat_v = pool_v.reshape(-1, D)
    want = {}
    for s in range(pager.bmax):
        if not pager.active[s]:
            continue
        for h in range(pager.hkv):
            L = int(pager.lengths[s, h])
            rows = np.array([pager.physical_row(s, h, t) for t in range(L)], dtype=np.int64)
            want[(s, h)] = (flat_k[rows] if L else np.zeros((0, D), np.uint16),
                            flat_v[rows] if L else np.zeros((0, D), np.uint16), rows)
    return want
