"""Integer model of the split-KV work plan.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The FlashMLA usage on the pages computes a tile-scheduler plan and a split
count once per decode step from the cache lengths, then reuses it for every
layer (FlashMLA release news, usage example); the SC11 note picks per-core
schemes by batch count and sequence length. The plan here is this library's
own, and this module states it from its definition, as intervals:

* Sequence b has pages_b = ceil(L_b / page) pages (0 if L_b <= 0).
* Lay the sequences with pages_b > 0 end to end on a cost line, each taking
  F + pages_b units: F units of fixed per-sequence overhead, then one unit per
  page. Sequence b starts at C_b; its page p sits at C_b + F + p.
* With T the total and q = max(1, ceil(T / n_slots)), slot s owns the cost
  units [s q, min((s+1) q, T)). A slot processes every page whose unit it owns;
  the pages of one sequence inside one slot form one piece (a split).
* splits_b counts the slots holding at least one page of b;
  num_splits[b+1] = num_splits[b] + splits_b; a piece of b in slot s has split
  index num_splits[b] + (s - first slot of b).
* tile_meta[s] = [b_begin, page_begin, b_end, page_end, split_begin, 0, 0, 0]:
  the first and last sequences the slot touches, the first page (inclusive) in
  b_begin and last page (exclusive) in b_end, and the split index of the piece
  of b_begin. A slot with no page is [0, 0, -1, 0, 0, 0, 0, 0].
"""
from __future__ import annotations

import numpy as np

META_WORDS = 8


def seq_pages(seqlens, page: int = 64) -> np.ndarray:
    L = np.asarray(seqlens, dtype=np.int64)
    p = (L + page - 1) // page
    p[L <= 0] = 0
    return p


def plan(seqlens, n_slots: int, fixed_cost: int, page: int = 64):
    """Return (tile_meta int32 [n_slots, 8], num_splits int32 [b+1], pieces).

    ``pieces`` lists (slot, b, page_lo, page_hi, split_index) in slot order.
    """
    assert n_slots >= 1 and fixed_cost >= 0
    pages = seq_pages(seqlens, page)
    B = pages.size
    F = int(fixed_cost)
    start = np.zeros(B, dtype=np.int64)
    T = 0
    for b in range(B):
        start[b] = T
        if pages[b] > 0:
            T += F + int(pages[b])
    q = max(1, -(-T // n_slots)) if T > 0 else 1
    first = np.zeros(B, dtype=np.int64)
    splits = np.zeros(B, dtype=np.int64)
    for b in range(B):
        if pages[b] > 0:
            first[b] = (start[b] + F) // q
            last = (start[b] + F + pages[b] - 1) // q
            splits[b] = last - first[b] + 1
    ns = np.zeros(B + 1, dtype=np.int64)
    ns[1:] = np.cumsum(splits)
    meta = np.zeros((n_slots, META_WORDS), dtype=np.int64)
    pieces = []
    for s in range(n_slots):
        lo, hi = s * q, min((s + 1) * q, T)
        mine = []
        for b in range(B):
            if pages[b] == 0:
                continue
            a = max(lo, start[b] + F)
            e = min(hi, start[b] + F + pages[b])
            if a < e:
                mine.append((b, int(a - start[b] - F), int(e - start[b] - F)))
        if not mine:
            meta[s] = [0, 0, -1, 0, 0, 0, 0, 0]
            continue
        for (b, plo, phi) in mine:
            pieces.append((s, b, plo, phi, int(ns[b] + (s - first[b]))))
        b0, p0, _ = mine[0]
        b1, _, p1 = mine[-1]
        meta[s] = [b0, p0, b1, p1, ns[b0] + (s - first[b0]), 0, 0, 0]
    return meta.astype(np.int32), ns.astype(np.int32), pieces


def max_splits_bound(b: int, n_slots: int) -> int:
    """Upper bound on sum_b splits_b: every slot boundary inside a sequence adds one split."""
    return b + n_slots
